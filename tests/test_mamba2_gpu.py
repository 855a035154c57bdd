"""GPU parity of the Mamba2 SSM heads (dims.ssm_heads = S > 0).

The P = d_inner / S channels of a head share Delta_t (the dt block of the
projection has S columns) and one scalar A, so the scan and the decode step
take one exp2 per (step, channel).  Compared with the oracle: prefill
(fp32 and bf16, few-row and 256x256-tile GEMMs, one channel per head, with
RoPE too), a KV-sharing consumer, the meta prefix, decode after prefill on
ring and linear caches, and consumer decode.
"""
from dataclasses import replace

import numpy as np
import pytest

from hybrid_attention_ssm_amd.configs import HYMBA_1P5B, TINY, PrefillWorkload
from hybrid_attention_ssm_amd.synth import prefill_inputs
from oracle import hymba_ref as ref
from tests.harness import TOL, np_of, rel_err, run_meta_prefix, run_prefill
from tests.test_decode_gpu import SMALL_BF16, _decode_steps
from tests.test_parity_gpu import _check_prefill

pytestmark = pytest.mark.gpu

TINY_M2 = replace(TINY, ssm_heads=8)                   # 16 channels per head
SMALL_M2 = replace(SMALL_BF16, ssm_heads=8)            # 64 channels per head
SMALL_P32 = replace(SMALL_BF16, ssm_heads=16)          # 32 channels per head


@pytest.mark.parametrize("B,n,window,is_global", [
    (2, 300, 100, False), (1, 64, 16, False), (1, 37, 16, False),
    (1, 200, 64, True),
    (2, 1100, 64, False)])    # with the 256x256-tile in-projection
def test_prefill_mamba2_32_channel_heads(B, n, window, is_global):
    """bf16, 32 channels per head, sequences of one partial chunk to many."""
    _check_prefill(SMALL_P32, B, n, window, is_global, seed=400 + n, cache_cap=128 if not is_global else 256)


def test_mamba2_hymba_shapes_100_heads():
    """The 1.5B layer widths with 100 heads of 32 channels."""
    _check_prefill(replace(HYMBA_1P5B, ssm_heads=100), 1, 333, 64, False, seed=8)


@pytest.mark.parametrize("dims,B,n,window,is_global,cap", [
    (TINY_M2, 2, 64, 16, False, 16), (TINY_M2, 1, 50, 16, True, 64),
    (replace(TINY, ssm_heads=128), 1, 40, 8, False, 8),                 # one channel per head
    (SMALL_M2, 1, 300, 100, False, 128), (replace(SMALL_BF16, ssm_heads=32), 2, 130, 64, True, 256),
    (SMALL_M2, 2, 600, 128, False, 128),                                # 256x256-tile GEMM
    (replace(SMALL_M2, rope_base=10000.0), 1, 200, 64, False, 128)])    # with RoPE too
def test_prefill_with_mamba2_heads(dims, B, n, window, is_global, cap):
    _check_prefill(dims, B, n, window, is_global, seed=300 + n, cache_cap=cap)


def test_mamba2_hymba_shapes():
    """The 1.5B layer widths with 64 heads of 50 channels."""
    _check_prefill(replace(HYMBA_1P5B, ssm_heads=64), 1, 200, 64, False, seed=6)


@pytest.mark.parametrize("dims", [TINY_M2, SMALL_M2])
def test_consumer_prefill_with_mamba2_heads(dims):
    B, n, window = 2, 90, 20
    wp = PrefillWorkload("p", 71, dims, B, n, window, False)
    ip = prefill_inputs(wp, varied=True)
    ic = prefill_inputs(replace(wp, seed=72), kv_producer=False, varied=True)
    pr = ref.prefill(dims.as_dict(), ip["weights"], ip["R"], ip["x"], window, False)
    cr = ref.prefill(dims.as_dict(), ic["weights"], ip["R"], ic["x"], window, False,
                     shared_kv=(pr["K_all"], pr["V_all"]))
    prod = run_prefill(dims, ip["weights"], ip["R"], ip["x"], window, False)
    cons = run_prefill(dims, ic["weights"], ip["R"], ic["x"], window, False, producer=prod)
    tol = TOL[dims.dtype]
    assert rel_err(np_of(cons["out"]), cr["out"]) <= tol
    assert rel_err(np_of(cons["h"]), cr["h"]) <= tol


@pytest.mark.parametrize("dims", [TINY_M2, SMALL_M2])
def test_meta_prefix_with_mamba2_heads(dims):
    inp = prefill_inputs(PrefillWorkload("m", 13, dims, 1, 8, 4, False), varied=True)
    _, meta = run_meta_prefix(dims, inp["weights"], inp["R"])
    want = ref.meta_prefix(dims.as_dict(), inp["weights"], inp["R"])
    tol = TOL[dims.dtype]
    assert rel_err(np_of(meta["h0"]), want["h0"]) <= tol
    assert rel_err(np_of(meta["conv_tail"]), want["conv_tail"]) <= tol


@pytest.mark.parametrize("dims,n0,steps,window,is_global,cap", [
    (TINY_M2, 10, 12, 8, False, 8), (TINY_M2, 20, 5, 16, True, 32),
    (SMALL_M2, 60, 9, 64, False, 64), (SMALL_M2, 130, 4, 64, True, 160),
    (SMALL_P32, 150, 6, 64, False, 64)])
def test_decode_with_mamba2_heads(dims, n0, steps, window, is_global, cap):
    B = 2
    inp = prefill_inputs(PrefillWorkload("pd", n0 + steps, dims, B, n0 + steps, window, is_global), varied=True)
    x = inp["x"]
    print(f"case {dims.dtype} S={dims.ssm_heads} n0={n0} steps={steps} global={is_global}", flush=True)
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
    assert rel_err(np_of(got["h"]), want["h"]) <= tol
    assert rel_err(np_of(got["conv"]), want["conv_tail"]) <= tol
