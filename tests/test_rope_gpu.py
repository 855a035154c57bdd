"""GPU parity of the rotary position embedding of Q and K (rope_base > 0).

The library turns Q and K inside the input projection's epilogue (the GEMM
reads each head's weight rows in pair order, so every 4-column group holds
two whole rotation pairs).  Compared with the oracle: prefill outputs and K
buffers (fp32 head_dim 32 and 64, bf16), a KV-sharing consumer, the meta
prefix (meta keys at positions 0..m-1), decode after prefill across a ring
wrap and on a linear cache (new token at m + len), and consumer decode (its
token at m + len - 1).
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from hybrid_attention_ssm_amd import binding as hb
from hybrid_attention_ssm_amd.configs import HYMBA_1P5B, TINY, PrefillWorkload
from hybrid_attention_ssm_amd.synth import prefill_inputs
from oracle import hymba_ref as ref
from tests.harness import TOL, np_of, rel_err, run_meta_prefix, run_prefill
from tests.test_decode_gpu import SMALL_BF16, _decode_steps
from tests.test_parity_gpu import _check_prefill

pytestmark = pytest.mark.gpu

TINY_R = replace(TINY, rope_base=10000.0)
TINY64_R = replace(TINY, d_model=128, n_heads=6, n_kv_heads=2, head_dim=64, d_inner=96,
                   n_meta=7, d_conv=3, rope_base=500.0)
SMALL_BF16_R = replace(SMALL_BF16, rope_base=10000.0)


@pytest.mark.parametrize("dims,B,n,window,is_global,cap", [
    (TINY_R, 2, 64, 16, False, 16), (TINY_R, 1, 50, 16, True, 64), (TINY64_R, 2, 45, 9, False, 12),
    (SMALL_BF16_R, 1, 300, 100, False, 128), (SMALL_BF16_R, 2, 130, 64, True, 256),
    (replace(SMALL_BF16, rope_base=500000.0), 1, 200, 64, False, 128),
    # 1024 rows or more: the 256x256-tile GEMM, whose lanes own both halves
    # of their pairs (the shorter cases take the few-row GEMM, which reads
    # the weight rows in pair order)
    (SMALL_BF16_R, 2, 600, 128, False, 128), (SMALL_BF16_R, 1, 1100, 64, True, 1200)])
def test_prefill_with_rope(dims, B, n, window, is_global, cap):
    _check_prefill(dims, B, n, window, is_global, seed=200 + n, cache_cap=cap)


def test_prefill_with_rope_hymba_shapes():
    _check_prefill(replace(HYMBA_1P5B, rope_base=10000.0), 1, 200, 64, False, seed=5)


def test_rope_changes_the_output():
    """The same inputs with and without RoPE give different outputs (the
    rotation is really applied, not silently dropped)."""
    _, want0, got0 = _check_prefill(SMALL_BF16, 1, 130, 64, False, seed=77)
    _, want1, got1 = _check_prefill(SMALL_BF16_R, 1, 130, 64, False, seed=77)
    assert rel_err(want1["out"], want0["out"]) > 0.1
    assert rel_err(np_of(got1["out"]), np_of(got0["out"])) > 0.1


@pytest.mark.parametrize("dims", [TINY_R, SMALL_BF16_R])
def test_consumer_prefill_with_rope(dims):
    B, n, window = 2, 90, 20
    wp = PrefillWorkload("p", 51, dims, B, n, window, False)
    ip = prefill_inputs(wp, varied=True)
    ic = prefill_inputs(replace(wp, seed=52), kv_producer=False, varied=True)
    pr = ref.prefill(dims.as_dict(), ip["weights"], ip["R"], ip["x"], window, False)
    cr = ref.prefill(dims.as_dict(), ic["weights"], ip["R"], ic["x"], window, False,
                     shared_kv=(pr["K_all"], pr["V_all"]))
    prod = run_prefill(dims, ip["weights"], ip["R"], ip["x"], window, False)
    cons = run_prefill(dims, ic["weights"], ip["R"], ic["x"], window, False, producer=prod)
    tol = TOL[dims.dtype]
    e = rel_err(np_of(cons["out"]), cr["out"])
    print(f"consumer err {e:.2e}", flush=True)
    assert e <= tol


@pytest.mark.parametrize("dims", [TINY_R, SMALL_BF16_R])
def test_meta_prefix_with_rope(dims):
    inp = prefill_inputs(PrefillWorkload("m", 9, dims, 1, 8, 4, False), varied=True)
    _, meta = run_meta_prefix(dims, inp["weights"], inp["R"])
    want = ref.meta_prefix(dims.as_dict(), inp["weights"], inp["R"])
    tol = TOL[dims.dtype]
    assert rel_err(np_of(meta["k"]), want["k"]) <= tol
    assert rel_err(np_of(meta["v"]), want["v"]) <= tol


@pytest.mark.parametrize("dims,n0,steps,window,is_global,cap", [
    (TINY_R, 10, 12, 8, False, 8), (TINY_R, 20, 5, 16, True, 32),
    (SMALL_BF16_R, 60, 9, 64, False, 64), (SMALL_BF16_R, 130, 4, 64, True, 160)])
def test_decode_with_rope(dims, n0, steps, window, is_global, cap):
    B = 2
    inp = prefill_inputs(PrefillWorkload("pd", n0 + steps, dims, B, n0 + steps, window, is_global), varied=True)
    x = inp["x"]
    print(f"case {dims.dtype} n0={n0} steps={steps} W={window} global={is_global}", flush=True)
    z = np.zeros((B, dims.n_kv_heads, cap, dims.head_dim))
    want = ref.prefill(dims.as_dict(), inp["weights"], inp["R"], x, window, is_global,
                       cache=dict(k=z, v=z, is_ring=not is_global))
    got = run_prefill(dims, inp["weights"], inp["R"], x[:, :n0], window, is_global,
                      cache_cap=cap, cache_ring=not is_global)
    outs = _decode_steps(dims, got, x[:, n0:], window, is_global, cap)
    tol = TOL[dims.dtype]
    for s, o in enumerate(outs):
        e = rel_err(o, want["out"][:, n0 + s])
        assert e <= tol, f"step {s}: {e}"
    assert rel_err(np_of(got["cache_k"]), want["cache_k"]) <= tol


@pytest.mark.parametrize("dims", [TINY_R, SMALL_BF16_R])
def test_consumer_decode_with_rope(dims):
    B, n0, steps, window = 2, 30, 6, 16
    cap = window
    wp = PrefillWorkload("p", 61, dims, B, n0 + steps, window, False)
    ip = prefill_inputs(wp, varied=True)
    ic = prefill_inputs(replace(wp, seed=62), kv_producer=False, varied=True)
    mp = ref.meta_prefix(dims.as_dict(), ip["weights"], ip["R"])
    z = np.zeros((B, dims.n_kv_heads, cap, dims.head_dim))
    pre_p = ref.prefill(dims.as_dict(), ip["weights"], ip["R"], ip["x"][:, :n0], window, False,
                        cache=dict(k=z, v=z, is_ring=True))
    pre_c = ref.prefill(dims.as_dict(), ic["weights"], ip["R"], ic["x"][:, :n0], window, False,
                        shared_kv=(pre_p["K_all"], pre_p["V_all"]))
    gp = run_prefill(dims, ip["weights"], ip["R"], ip["x"][:, :n0], window, False, cache_cap=cap)
    gc = run_prefill(dims, ic["weights"], ip["R"], ic["x"][:, :n0], window, False, producer=gp)
    outs = _decode_steps(dims, gp, ip["x"][:, n0:], window, False, cap,
                         consumer=(gc["layer"], gc["h"], gc["conv"], ic["x"][:, n0:]))
    cache = dict(k=pre_p["cache_k"], v=pre_p["cache_v"], len=np.full(B, n0), is_ring=True)
    hp, cp, hc, cc = pre_p["h"], pre_p["conv_tail"], pre_c["h"], pre_c["conv_tail"]
    tol = TOL[dims.dtype]
    for s in range(steps):
        rp = ref.decode_step(dims.as_dict(), ip["weights"], ip["x"][:, n0 + s], mp["k"], mp["v"],
                             window, False, cache, hp, cp)
        cache = dict(k=rp["cache_k"], v=rp["cache_v"], len=rp["len"], is_ring=True)
        rc = ref.decode_step(dims.as_dict(), ic["weights"], ic["x"][:, n0 + s], mp["k"], mp["v"],
                             window, False, cache, hc, cc)
        hp, cp, hc, cc = rp["h"], rp["conv"], rc["h"], rc["conv"]
        assert rel_err(outs[s][0], rp["out"]) <= tol
        assert rel_err(outs[s][1], rc["out"]) <= tol
