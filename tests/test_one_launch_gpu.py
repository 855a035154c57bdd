"""GPU: the attention and scan pass 3 in one launch (bf16, opt-in).

With HH_ONE_LAUNCH_BRANCHES=1 hh_prefill runs scan passes 1 and 2, then one
grid whose workgroups are either attention workgroups or groups of scan
pass-3 waves; by default (0) the attention kernel runs, then the scan's
passes with its own pass-3 kernel.  Both run the same device code on the same
inputs, so every output, state, conv history, K/V buffer and cache length
must agree bit for bit; the one-launch run is also compared with the oracle.

The shapes cover every way a scan workgroup can be filled: 5, 4 and 8 waves
per workgroup (4 of them scanning, the rest ending at once), a channel count
that leaves the last group with 3 of 4 blocks, several sequences, a single
chunk, the fused norm (1024 rows or more) and the separate norm kernel, Mamba
and Mamba2 heads, sliding-window and global layers.
"""
from dataclasses import replace

import pytest
import torch

from hybrid_attention_ssm_amd.configs import HYMBA_1P5B, PrefillWorkload
from hybrid_attention_ssm_amd.synth import prefill_inputs
from oracle import hymba_ref as ref
from tests.harness import TOL, np_of, rel_err, run_prefill
from tests.test_decode_gpu import SMALL_BF16

pytestmark = pytest.mark.gpu

KEYS = ("out", "h", "conv", "full_k", "full_v", "cache_k", "cache_v", "len")

CASES = [
    # dims, B, n, window, is_global, cache cap
    (HYMBA_1P5B, 1, 1100, 1024, False, 1024),                          # 5 waves, fused norm
    (HYMBA_1P5B, 1, 600, 256, False, 256),                             # 5 waves, separate norm
    (SMALL_BF16, 2, 700, 64, False, 64),                               # 4 waves, two sequences
    (replace(SMALL_BF16, d_inner=448), 1, 1030, 48, True, 1030),       # 7 channel blocks, global
    (replace(SMALL_BF16, n_kv_heads=1), 1, 520, 100, False, 100),      # 8 waves per workgroup
    (replace(SMALL_BF16, ssm_heads=8, rope_base=10000.0), 2, 560, 100, False, 128),   # Mamba2 heads
    (SMALL_BF16, 1, 40, 16, False, 16),                                # one chunk
]
IDS = ["1.5B-fused", "1.5B-separate", "bf16-b2", "bf16-448ch-global", "bf16-8waves", "bf16-mamba2-rope",
       "bf16-one-chunk"]


@pytest.mark.parametrize("dims,B,n,window,is_global,cap", CASES, ids=IDS)
def test_one_launch_matches_two_launches(dims, B, n, window, is_global, cap, monkeypatch):
    print(f"case one-launch d={dims.d_model} H={dims.n_heads}/{dims.n_kv_heads} D={dims.d_inner} "
          f"S={dims.ssm_heads} B={B} n={n} W={window} global={is_global}", flush=True)
    inp = prefill_inputs(PrefillWorkload("ol", 700 + n, dims, B, n, window, is_global), varied=True)
    runs = {}
    for mode in ("0", "1"):
        monkeypatch.setenv("HH_ONE_LAUNCH_BRANCHES", mode)
        runs[mode] = run_prefill(dims, inp["weights"], inp["R"], inp["x"], window, is_global,
                                 cache_cap=cap, cache_ring=not is_global)
    two, one = runs["0"], runs["1"]
    for key in KEYS:
        assert torch.equal(two[key], one[key]), key
    want = ref.prefill(dims.as_dict(), inp["weights"], inp["R"], inp["x"], window, is_global)
    tol = TOL[dims.dtype]
    e_out, e_h = rel_err(np_of(one["out"]), want["out"]), rel_err(np_of(one["h"]), want["h"])
    print(f"  err out={e_out:.2e} h={e_h:.2e}", flush=True)
    assert e_out <= tol and e_h <= tol


def test_one_launch_repeated_calls(monkeypatch):
    """Back-to-back prefills in one launch each: the scan workgroups borrow
    the attention's LDS arrays, so nothing may leak from one call (or one
    workgroup) into the next."""
    monkeypatch.setenv("HH_ONE_LAUNCH_BRANCHES", "1")
    dims = SMALL_BF16
    B, n, W = 1, 1200, 64
    print(f"case one-launch repeated B={B} n={n}", flush=True)
    inp = prefill_inputs(PrefillWorkload("olr", 77, dims, B, n, W, False), varied=True)
    first = run_prefill(dims, inp["weights"], inp["R"], inp["x"], W, False, cache_cap=W)
    for _ in range(2):
        again = run_prefill(dims, inp["weights"], inp["R"], inp["x"], W, False, cache_cap=W)
        for key in KEYS:
            assert torch.equal(first[key], again[key]), key
