"""GPU parity of the fusion step folded into the output projection.

For bf16 prefills of 1024 rows or more the RMSNorm, beta scaling and average
of Eq. (3) (Hymba paper, §2.1) run without a kernel of their own: the
attention and scan kernels store beta-scaled branch outputs together with
per-row sums of squares of the unscaled ones, and the output projection
multiplies its accumulators by the per-row factors 1/(2 rms).  HH_FUSED_NORM=0
selects the separate norm kernel for the same call.

Both paths are compared with the oracle at the layer's bf16 bar.  The SSM
state, conv tail, K/V and cache contents do not depend on the path and must
agree bit for bit; the cache length, which the fused path's attention kernel
records, must equal the prompt length.  Row counts are ragged with respect to
both GEMM row tiles (256) and the scan's chunks, and the shapes select both
GEMM tile shapes (256x256 for d_model 256, 256x224 for d_model 1600).
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from hybrid_attention_ssm_amd.configs import HYMBA_1P5B, LayerDims, PrefillWorkload
from hybrid_attention_ssm_amd.synth import prefill_inputs
from oracle import hymba_ref as ref
from tests.harness import TOL, np_of, rel_err, run_prefill

pytestmark = pytest.mark.gpu

SMALL_BF16 = LayerDims(d_model=256, n_heads=8, n_kv_heads=2, head_dim=64, d_inner=512,
                       d_state=16, d_conv=4, n_meta=128, dtype="bf16")

STATE_KEYS = ("h", "conv", "full_k", "full_v", "cache_k", "cache_v", "len")


def _run_both(monkeypatch, dims, inp, window, is_global, cache_cap, producer=None):
    runs = {}
    for mode in ("1", "0"):
        monkeypatch.setenv("HH_FUSED_NORM", mode)
        runs[mode] = run_prefill(dims, inp["weights"], inp["R"], inp["x"], window, is_global,
                                 producer=producer, cache_cap=cache_cap, cache_ring=not is_global)
    return runs["1"], runs["0"]


@pytest.mark.parametrize("dims,B,n,window,is_global,seed", [
    (SMALL_BF16, 2, 640, 16, False, 301),
    (SMALL_BF16, 1, 1100, 48, True, 302),
    (HYMBA_1P5B, 1, 1040, 1024, False, 303),
], ids=["small-swa-B2", "small-global", "1.5B-swa"])
def test_fused_norm_matches_oracle_and_separate_norm(monkeypatch, dims, B, n, window, is_global, seed):
    print(f"case fused norm d={dims.d_model} B={B} n={n} W={window} global={is_global} seed={seed}",
          flush=True)
    assert B * n >= 1024
    inp = prefill_inputs(PrefillWorkload("fused", seed, dims, B, n, window, is_global), varied=True)
    cap = n if is_global else window
    z = np.zeros((B, dims.n_kv_heads, cap, dims.head_dim))
    want = ref.prefill(dims.as_dict(), inp["weights"], inp["R"], inp["x"], window, is_global,
                       cache=dict(k=z, v=z, is_ring=not is_global))
    fused, sep = _run_both(monkeypatch, dims, inp, window, is_global, cap)
    tol = TOL[dims.dtype]
    e_f, e_s = rel_err(np_of(fused["out"]), want["out"]), rel_err(np_of(sep["out"]), want["out"])
    e_fs = rel_err(np_of(fused["out"]), np_of(sep["out"]).astype(np.float64))
    print(f"  err out fused={e_f:.2e} separate={e_s:.2e} fused-vs-separate={e_fs:.2e}", flush=True)
    assert e_f <= tol and e_s <= tol
    for k in STATE_KEYS:
        assert torch.equal(fused[k], sep[k]), k
    assert (fused["len"].cpu().numpy() == n).all()


def test_fused_norm_consumer_layer(monkeypatch):
    """A KV-sharing consumer (no K/V columns, no cache of its own) on the
    fused path, reading its producer's keys and values."""
    dims = SMALL_BF16
    B, n, W = 1, 1500, 32
    print(f"case fused norm consumer B={B} n={n} W={W}", flush=True)
    wp = PrefillWorkload("fp", 304, dims, B, n, W, False)
    inp_p = prefill_inputs(wp, varied=True)
    inp_c = prefill_inputs(replace(wp, seed=305), kv_producer=False, varied=True)
    prod_ref = ref.prefill(dims.as_dict(), inp_p["weights"], inp_p["R"], inp_p["x"], W, False)
    want = ref.prefill(dims.as_dict(), inp_c["weights"], inp_p["R"], inp_c["x"], W, False,
                       shared_kv=(prod_ref["K_all"], prod_ref["V_all"]))
    monkeypatch.setenv("HH_FUSED_NORM", "1")
    prod = run_prefill(dims, inp_p["weights"], inp_p["R"], inp_p["x"], W, False)
    got = run_prefill(dims, inp_c["weights"], inp_p["R"], inp_c["x"], W, False, producer=prod)
    tol = TOL[dims.dtype]
    e, e_h = rel_err(np_of(got["out"]), want["out"]), rel_err(np_of(got["h"]), want["h"])
    print(f"  err out={e:.2e} h={e_h:.2e}", flush=True)
    assert e <= tol and e_h <= tol
