"""GPU parity of the stage hooks: each branch's prefill kernels on inputs of
their own, against the oracle's definition of that branch.

* hh_stage_attn: the attention heads of Hymba paper §2.1 Eq. (1) over the meta
  keys (§2.3) and the sliding window or the causal prefix (§2.2), compared
  with the oracle's per-query softmax over exactly the allowed rows.
* hh_stage_ssm: the SSM heads of Eq. (2) (causal conv + SiLU, selective scan
  from a given state, SiLU gate), compared with the oracle's conv, its
  literal recurrence and gate; the final state and the conv history too.
  Mamba heads and Mamba2 heads (scalar decay per head), with and without a
  starting state.

Sizes span several scan chunks, several key tiles and ragged tails.  O and Y
are stored in the storage type, so each element is allowed its own rounding
to that type (unit roundoff times its magnitude) before the RMS-relative bar:
with random unit-variance inputs O has heavy tails, and bf16 rounding alone
moves its largest elements by 2.8% of its RMS.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from hybrid_attention_ssm_amd import binding as hb
from hybrid_attention_ssm_amd.configs import TINY, LayerDims
from hybrid_attention_ssm_amd.synth import attn_stage_inputs, layer_weights, ssm_stage_inputs
from oracle import hymba_ref as ref
from tests.harness import (TOL, assert_written, check_guards, guarded, np_of, poisoned_workspace, rel_err,
                           rel_err_stored)

pytestmark = pytest.mark.gpu

SMALL_BF16 = LayerDims(d_model=256, n_heads=8, n_kv_heads=2, head_dim=64, d_inner=512,
                       d_state=16, d_conv=4, n_meta=128, dtype="bf16")


@pytest.mark.parametrize("dims,B,n,W,is_global,seed", [
    (TINY, 2, 70, 16, False, 401),
    (TINY, 1, 90, 16, True, 402),
    (SMALL_BF16, 2, 200, 48, False, 403),
    (SMALL_BF16, 1, 150, 48, True, 404),
    (replace(SMALL_BF16, n_meta=0), 1, 97, 32, False, 405),
], ids=["f32-swa", "f32-global", "bf16-swa", "bf16-global", "bf16-no-meta"])
def test_stage_attn_matches_oracle(dims, B, n, W, is_global, seed):
    print(f"case stage_attn {dims.dtype} m={dims.n_meta} B={B} n={n} W={W} global={is_global}", flush=True)
    inp = attn_stage_inputs(dims, B, n, seed)
    sd = hb.storage_dtype(dims)
    H, G, hd, m = dims.n_heads, dims.n_kv_heads, dims.head_dim, dims.n_meta
    dev = {k: hb.to_device(v, sd) for k, v in inp.items()}
    o = guarded((B, n, H * hd), sd)
    hb.hh_stage_attn(dims, dev["q"], dev["k"], dev["v"], dev["meta_k"] if m else None,
                     dev["meta_v"] if m else None, W, is_global, o)
    torch.cuda.synchronize()
    assert_written("o", o)
    check_guards()
    got = np_of(o)
    want = np.empty((B, n, H * hd))
    scale = 1.0 / np.sqrt(hd)
    q = inp["q"].astype(np.float64)
    for b in range(B):
        K = np.concatenate([inp["meta_k"].transpose(1, 0, 2), inp["k"][b].transpose(1, 0, 2)]).astype(np.float64)
        V = np.concatenate([inp["meta_v"].transpose(1, 0, 2), inp["v"][b].transpose(1, 0, 2)]).astype(np.float64)
        for p in range(n):
            rows = ref.allowed_rows(m + p, m, W, is_global)
            want[b, p] = ref.attend(q[b, p].reshape(H, hd), K, V, rows, scale)[0].reshape(-1)
    e = rel_err_stored(got, want, dims.dtype)   # O is stored in the storage type
    print(f"  err o={e:.2e} (plain rel_err {rel_err(got, want):.2e})", flush=True)
    assert e <= TOL[dims.dtype]


def _block_major(a: np.ndarray) -> np.ndarray:
    """[R, C] -> element (r, c) at ((c/64) R + r) 64 + c%64 (whole 64-column blocks)."""
    R, C = a.shape
    C64 = (C + 63) // 64 * 64
    p = np.zeros((R, C64), a.dtype)
    p[:, :C] = a
    return np.ascontiguousarray(p.reshape(R, C64 // 64, 64).transpose(1, 0, 2)).reshape(-1)


@pytest.mark.parametrize("dims,B,n,with_state,seed", [
    (TINY, 2, 70, True, 411),
    (SMALL_BF16, 2, 300, True, 412),
    (SMALL_BF16, 1, 1000, False, 413),
    (replace(SMALL_BF16, ssm_heads=8), 2, 260, True, 414),
    (replace(TINY, ssm_heads=4), 1, 130, False, 415),
], ids=["f32", "bf16", "bf16-zero-start", "bf16-mamba2", "f32-mamba2-zero-start"])
def test_stage_ssm_matches_oracle(dims, B, n, with_state, seed):
    print(f"case stage_ssm {dims.dtype} S={dims.ssm_heads} B={B} n={n} state={with_state}", flush=True)
    inp = ssm_stage_inputs(dims, B, n, seed)
    sd = hb.storage_dtype(dims)
    D, N, k, R = dims.d_inner, dims.d_state, dims.d_conv, B * n
    w = layer_weights(np.random.default_rng(seed + 1000), dims)
    w.update(A=inp["A"], conv_w=inp["conv_w"], conv_b=inp["conv_b"])
    layer = hb.upload_weights(dims, w)
    f32 = torch.float32
    xs = hb.to_device(_block_major(inp["xs"]), f32)
    z = hb.to_device(_block_major(inp["z"]), sd)
    delta = hb.to_device(_block_major(inp["delta"]), f32)
    bc = hb.to_device(inp["bc"], f32)
    h0 = hb.to_device(inp["h0"], f32) if with_state else None
    tail0 = hb.to_device(inp["conv_tail"], f32) if with_state else None
    y = guarded((R, D), sd)
    h = guarded((B, D, N), f32)
    tail = guarded((B, k - 1, D), f32)
    ws = poisoned_workspace(hb.hh_stage_ssm_workspace_size(dims, B, n))
    hb.hh_stage_ssm(layer, xs, z, delta, bc, h0, tail0, B, n, y, h, tail, ws=ws)
    torch.cuda.synchronize()
    for name, t in (("y", y), ("h", h), ("tail", tail)):
        assert_written(name, t)
    check_guards()
    want_y = np.empty((R, D))
    want_h = np.empty((B, D, N))
    want_tail = np.empty((B, k - 1, D))
    hist = inp["conv_tail"].astype(np.float64) if with_state else np.zeros((k - 1, D))
    hstart = inp["h0"].astype(np.float64) if with_state else np.zeros((D, N))
    wd = {kk: (v.astype(np.float64) if isinstance(v, np.ndarray) else v) for kk, v in inp.items()}
    for b in range(B):
        r = slice(b * n, (b + 1) * n)
        u = ref.silu(ref.causal_conv(wd["xs"][r], wd["conv_w"], wd["conv_b"], hist))
        delta_c, A_c = ref.ssm_params(wd["delta"][r], wd["A"], dims.as_dict())
        yy, hh = ref.selective_scan(u, delta_c, A_c, wd["bc"][r, :N], wd["bc"][r, N:], hstart)
        want_y[r] = yy * ref.silu(wd["z"][r])
        want_h[b] = hh
        want_tail[b] = np.concatenate([hist, wd["xs"][r]])[-(k - 1):]
    tol = TOL[dims.dtype]
    e_y = rel_err_stored(np_of(y), want_y, dims.dtype)   # Y is stored in the storage type
    e_h, e_t = rel_err(np_of(h), want_h), rel_err(np_of(tail), want_tail)
    print(f"  err y={e_y:.2e} h={e_h:.2e} tail={e_t:.2e}", flush=True)
    assert e_y <= tol and e_h <= tol and e_t <= tol
