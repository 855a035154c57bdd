"""GPU parity on the degenerate and ragged cases of the layer.

* No meta tokens (m = 0): attention over real keys only, the SSM from a zero
  state (the layer without the meta-token part of the paper's §2.3).
* Decode over a batch whose sequences hold different numbers of positions
  (1 to several windows, some not yet wrapped), for a ring (SWA producer and
  KV-sharing consumer) and a linear (global) cache, on both bf16 decode
  attention kernels (meta count a multiple of 32 and not) and the fp32 one.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from hybrid_attention_ssm_amd import binding as hb
from hybrid_attention_ssm_amd.configs import (TINY, DecodeLayer, DecodeWorkload, LayerDims,
                                              PrefillWorkload)
from hybrid_attention_ssm_amd.synth import decode_inputs, prefill_inputs
from oracle import hymba_ref as ref
from tests.harness import TOL, np_of, rel_err, run_prefill

pytestmark = pytest.mark.gpu

SMALL_BF16 = LayerDims(d_model=256, n_heads=8, n_kv_heads=2, head_dim=64, d_inner=512,
                       d_state=16, d_conv=4, n_meta=128, dtype="bf16")


@pytest.mark.parametrize("dims", [replace(TINY, n_meta=0), replace(SMALL_BF16, n_meta=0)],
                         ids=["f32", "bf16"])
@pytest.mark.parametrize("is_global", [False, True], ids=["swa", "global"])
def test_no_meta_tokens_prefill(dims, is_global):
    B, n, W = 2, 77, 20
    inp = prefill_inputs(PrefillWorkload("nometa", 51, dims, B, n, W, is_global), varied=True)
    assert inp["R"].shape[0] == 0
    cap = n if is_global else W
    want = ref.prefill(dims.as_dict(), inp["weights"], inp["R"], inp["x"], W, is_global,
                       cache=dict(k=np.zeros((B, dims.n_kv_heads, cap, dims.head_dim)),
                                  v=np.zeros((B, dims.n_kv_heads, cap, dims.head_dim)),
                                  is_ring=not is_global))
    got = run_prefill(dims, inp["weights"], inp["R"], inp["x"], W, is_global, cache_cap=cap,
                      cache_ring=not is_global)
    tol = TOL[dims.dtype]
    errs = dict(out=rel_err(np_of(got["out"]), want["out"]), h=rel_err(np_of(got["h"]), want["h"]),
                conv=rel_err(np_of(got["conv"]), want["conv_tail"]),
                cache_k=rel_err(np_of(got["cache_k"]), want["cache_k"]))
    print(f"m=0 {dims.dtype} global={is_global}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
          flush=True)
    assert max(errs.values()) <= tol


def _ragged_decode(dims, lens, window, gcap, seed):
    """One decode step of an SWA producer, its consumer and a global producer
    over caches whose sequences hold `lens` positions; GPU against oracle."""
    B = len(lens)
    w = DecodeWorkload("ragged", seed, dims, batch=B, context=0, window=window, global_cap=gcap,
                       layers=(DecodeLayer(False, True, "swa"), DecodeLayer(False, False, "swa"),
                               DecodeLayer(True, True, "global")))
    inp = decode_inputs(w, varied=True)
    for c in inp["caches"].values():
        c["len"] = np.array(lens, np.int32)
    sd = hb.storage_dtype(dims)
    dev = {}
    for name, c in inp["caches"].items():
        kk, vv = hb.to_device(c["k"], sd), hb.to_device(c["v"], sd)
        ln = hb.to_device(c["len"], torch.int32)
        mk, mv = hb.to_device(c["meta_k"], sd), hb.to_device(c["meta_v"], sd)
        dev[name] = dict(k=kk, v=vv, len=ln, mk=mk, mv=mv, k0=kk.clone(), v0=vv.clone(),
                         kv=hb.make_kv(None, None, kk, vv, ln, c["cap"], c["is_ring"]),
                         meta=hb.make_meta(mk, mv, None, None))
    ocache = {name: dict(k=c["k"].astype(np.float64), v=c["v"].astype(np.float64), len=c["len"],
                         is_ring=c["is_ring"]) for name, c in inp["caches"].items()}
    tol = TOL[dims.dtype]
    for i, lay in enumerate(inp["layers"]):
        spec = lay["spec"]
        c = dev[spec.cache]
        layer = hb.upload_weights(dims, lay["weights"])
        h = hb.to_device(lay["h"], torch.float32)
        cv = hb.to_device(lay["conv"], torch.float32)
        out = torch.empty(B, dims.d_model, dtype=sd, device="cuda")
        hb.hh_decode_step(layer, hb.to_device(lay["x_t"], sd), c["meta"], window, spec.is_global,
                          c["kv"], h, cv, out)
        torch.cuda.synchronize()
        src = inp["caches"][spec.cache]
        r = ref.decode_step(dims.as_dict(), lay["weights"], lay["x_t"], src["meta_k"], src["meta_v"],
                            window, spec.is_global, ocache[spec.cache], lay["h"], lay["conv"])
        e_out, e_h = rel_err(np_of(out), r["out"]), rel_err(np_of(h), r["h"])
        e_c = rel_err(np_of(cv), r["conv"])
        print(f"  layer {i} ({spec.cache}, producer={spec.kv_producer}) out={e_out:.2e} "
              f"h={e_h:.2e} conv={e_c:.2e}", flush=True)
        assert max(e_out, e_h, e_c) <= tol
        if spec.kv_producer:
            ocache[spec.cache] = dict(k=r["cache_k"], v=r["cache_v"], len=r["len"],
                                      is_ring=src["is_ring"])
    for name, c in dev.items():
        o = ocache[name]
        assert (c["len"].cpu().numpy() == o["len"]).all()
        cap = inp["caches"][name]["cap"]
        for b, p in enumerate(lens):
            slot = p % cap if inp["caches"][name]["is_ring"] else p
            if slot < cap:   # the appended slot matches, every other slot is unchanged
                assert rel_err(np_of(c["k"][b][:, slot]), o["k"][b][:, slot]) <= tol
                mask = torch.ones(cap, dtype=torch.bool, device="cuda")
                mask[slot] = False
                assert torch.equal(c["k"][b][:, mask], c["k0"][b][:, mask])
                assert torch.equal(c["v"][b][:, mask], c["v0"][b][:, mask])


@pytest.mark.parametrize("dims", [TINY, SMALL_BF16, replace(SMALL_BF16, n_meta=70),
                                  replace(SMALL_BF16, n_meta=0),
                                  replace(TINY, rope_base=10000.0), replace(SMALL_BF16, rope_base=10000.0),
                                  replace(SMALL_BF16, ssm_heads=8, rope_base=500.0)],
                         ids=["f32", "bf16-m128", "bf16-m70", "bf16-m0", "f32-rope", "bf16-rope",
                              "bf16-mamba2-rope"])
def test_ragged_lengths_decode(dims):
    """Sequences at positions 1..45 in one batch: a ring of 16 (some not yet
    full, some wrapped several times) and a linear cache of 64."""
    lens = [1, 2, 15, 16, 17, 33, 45]
    print(f"ragged decode {dims.dtype} m={dims.n_meta}", flush=True)
    _ragged_decode(dims, lens, window=16, gcap=64, seed=61)


WIDE_BF16 = LayerDims(d_model=128, n_heads=2, n_kv_heads=1, head_dim=64, d_inner=4160, d_state=16, d_conv=4,
                      n_meta=4, dtype="bf16")


@pytest.mark.parametrize("dims,fused_norm", [
    # fp32 rows wider than 512 four-wide chunks and bf16 rows wider than 512
    # eight-wide chunks, with at least 2048 rows: the norm kernel that keeps
    # no row in registers (bf16 with the fusion step as its own kernel,
    # HH_FUSED_NORM=0; the default runs it inside the output projection)
    (LayerDims(d_model=64, n_heads=2, n_kv_heads=1, head_dim=32, d_inner=2560, d_state=16, d_conv=4,
               n_meta=4, dtype="f32"), "1"),
    (WIDE_BF16, "0"),
    (WIDE_BF16, "1")], ids=["f32-D2560", "bf16-D4160-norm-kernel", "bf16-D4160-fused"])
def test_wide_ssm_branch_many_rows(dims, fused_norm, monkeypatch):
    monkeypatch.setenv("HH_FUSED_NORM", fused_norm)
    n, W = 2048, 16
    print(f"case wide SSM {dims.dtype} D={dims.d_inner} n={n} HH_FUSED_NORM={fused_norm}", flush=True)
    inp = prefill_inputs(PrefillWorkload("wide", 52, dims, 1, n, W, False), varied=True)
    want = ref.prefill(dims.as_dict(), inp["weights"], inp["R"], inp["x"], W, False)
    got = run_prefill(dims, inp["weights"], inp["R"], inp["x"], W, False)
    tol = TOL[dims.dtype]
    e_out, e_h = rel_err(np_of(got["out"]), want["out"]), rel_err(np_of(got["h"]), want["h"])
    print(f"  err out={e_out:.2e} h={e_h:.2e}", flush=True)
    assert e_out <= tol and e_h <= tol


def test_injected_launch_failure_leaves_state_untouched(monkeypatch):
    """A launch failure of a decode step's first stage (injected on the host
    with HH_FAULT_INJECT) returns HH_ERR_HIP before anything is enqueued: the
    cache, its lengths, the SSM state and the output keep every bit.  An
    injected failure at a later stage is reported the same way."""
    dims = SMALL_BF16
    w = DecodeWorkload("inject", 62, dims, batch=3, context=0, window=16, global_cap=64,
                       layers=(DecodeLayer(False, True, "swa"),))
    inp = decode_inputs(w, varied=True)
    c = inp["caches"]["swa"]
    c["len"] = np.array([3, 20, 40], np.int32)
    sd = hb.storage_dtype(dims)
    kk, vv = hb.to_device(c["k"], sd), hb.to_device(c["v"], sd)
    ln = hb.to_device(c["len"], torch.int32)
    mk, mv = hb.to_device(c["meta_k"], sd), hb.to_device(c["meta_v"], sd)
    kv = hb.make_kv(None, None, kk, vv, ln, c["cap"], True)
    meta = hb.make_meta(mk, mv, None, None)
    lay = inp["layers"][0]
    layer = hb.upload_weights(dims, lay["weights"])
    h = hb.to_device(lay["h"], torch.float32)
    cv = hb.to_device(lay["conv"], torch.float32)
    out = torch.full((3, dims.d_model), 7.0, dtype=sd, device="cuda")
    before = [t.clone() for t in (kk, vv, ln, h, cv, out)]
    xt = hb.to_device(lay["x_t"], sd)
    monkeypatch.setenv("HH_FAULT_INJECT", "decode_inproj")
    with pytest.raises(hb.HHError) as ei:
        hb.hh_decode_step(layer, xt, meta, w.window, False, kv, h, cv, out)
    assert ei.value.status == 4 and "injected" in str(ei.value)
    torch.cuda.synchronize()
    for a, b in zip((kk, vv, ln, h, cv, out), before):
        assert torch.equal(a, b)
    monkeypatch.setenv("HH_FAULT_INJECT", "decode_norm")
    with pytest.raises(hb.HHError) as ei:
        hb.hh_decode_step(layer, xt, meta, w.window, False, kv, h, cv, out)
    assert ei.value.status == 4 and "decode_norm" in str(ei.value)
    torch.cuda.synchronize()
    monkeypatch.delenv("HH_FAULT_INJECT")
