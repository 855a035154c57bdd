"""hh_decode_step_noalloc: the decode step for callers that cannot allocate
(its scratch is the library's static per-GPU array) against hh_decode_step
with a caller workspace, through the C ABI.

Two calls in a row on the same GPU, the second with a smaller batch, each on
copies of the same caches and states; both entry points run the same
kernels, so outputs, states, caches and lengths must agree bit for bit.  A
step that needs more scratch than the static array holds is rejected before
anything is enqueued.
"""
import ctypes

import numpy as np
import pytest
import torch

from hybrid_attention_ssm_amd import binding as hb
from hybrid_attention_ssm_amd.configs import (HYMBA_1P5B, TINY, DecodeLayer, DecodeWorkload,
                                              LayerDims)
from hybrid_attention_ssm_amd.synth import decode_inputs

SMALL_BF16 = LayerDims(d_model=256, n_heads=8, n_kv_heads=2, head_dim=64, d_inner=512,
                       d_state=16, d_conv=4, n_meta=128, dtype="bf16")
LAYERS = (DecodeLayer(False, True, "swa"), DecodeLayer(False, False, "swa"),
          DecodeLayer(True, True, "global"))


def _device_copy(inp, dims):
    sd = hb.storage_dtype(dims)
    caches = {}
    for name, c in inp["caches"].items():
        kk, vv = hb.to_device(c["k"], sd), hb.to_device(c["v"], sd)
        ln = hb.to_device(c["len"], torch.int32)
        mk, mv = hb.to_device(c["meta_k"], sd), hb.to_device(c["meta_v"], sd)
        caches[name] = dict(k=kk, v=vv, len=ln, mk=mk, mv=mv,
                            kv=hb.make_kv(None, None, kk, vv, ln, c["cap"], c["is_ring"]),
                            meta=hb.make_meta(mk, mv, None, None))
    states = [(hb.to_device(l["h"], torch.float32), hb.to_device(l["conv"], torch.float32))
              for l in inp["layers"]]
    return caches, states


def _run(dims, inp, w, noalloc):
    sd = hb.storage_dtype(dims)
    caches, states = _device_copy(inp, dims)
    outs = []
    for lay, (h, cv) in zip(inp["layers"], states):
        spec = lay["spec"]
        c = caches[spec.cache]
        layer = hb.upload_weights(dims, lay["weights"])
        out = torch.full((w.batch, dims.d_model), float("nan"), dtype=sd, device="cuda")
        xt = hb.to_device(lay["x_t"], sd)
        if noalloc:
            hb.hh_decode_step_noalloc(layer, xt, c["meta"], w.window, spec.is_global, c["kv"], h, cv, out)
        else:
            hb.hh_decode_step(layer, xt, c["meta"], w.window, spec.is_global, c["kv"], h, cv, out)
        outs.append(out)
    torch.cuda.synchronize()
    return outs, states, caches


@pytest.mark.gpu
def test_noalloc_decode_matches_workspace_decode():
    # first call: 7 sequences on bf16 shapes (split attention, merged in the
    # norm); second call: a smaller batch of 3, fp32 shapes
    cases = [(SMALL_BF16, 7, [1, 2, 15, 16, 17, 33, 45], 91), (TINY, 3, [5, 16, 40], 92)]
    for dims, B, lens, seed in cases:
        print(f"case noalloc {dims.dtype} B={B}", flush=True)
        w = DecodeWorkload("noalloc", seed, dims, batch=B, context=0, window=16, global_cap=64, layers=LAYERS)
        inp = decode_inputs(w, varied=True)
        for c in inp["caches"].values():
            c["len"] = np.array(lens, np.int32)
        ref_out, ref_states, ref_caches = _run(dims, inp, w, noalloc=False)
        got_out, got_states, got_caches = _run(dims, inp, w, noalloc=True)
        for i in range(len(LAYERS)):
            assert not torch.isnan(got_out[i].float()).any()
            assert torch.equal(got_out[i], ref_out[i]), f"layer {i} out"
            assert torch.equal(got_states[i][0], ref_states[i][0]), f"layer {i} h"
            assert torch.equal(got_states[i][1], ref_states[i][1]), f"layer {i} conv"
        for name in ref_caches:
            for key in ("k", "v", "len"):
                assert torch.equal(got_caches[name][key], ref_caches[name][key]), f"{name} {key}"


def test_noalloc_rejects_a_step_beyond_the_static_scratch():
    """Batch 4096 at 1.5B widths needs more than the static scratch: the call
    fails with HH_ERR_WORKSPACE before touching a pointer (fake ones here)."""
    fake = 0x10000
    assert hb.hh_decode_workspace_size(HYMBA_1P5B, 4096, 8192) > (32 << 20)
    d = hb.hh_dims(HYMBA_1P5B)
    wts = hb.HHWeights(fake, fake, fake, fake, fake, fake, fake, fake, 1)
    meta = hb.HHMeta(fake, fake, fake, fake)
    st = hb.HHSsmState(fake, fake)
    kv = hb.HHKV(None, None, fake, fake, fake, 8192, 0)
    r = hb.lib().hh_decode_step_noalloc(ctypes.byref(d), ctypes.byref(wts), fake, 4096, ctypes.byref(meta),
                                        1024, 1, ctypes.byref(kv), ctypes.byref(st), fake, None)
    assert r == 3
    assert "static scratch" in hb.hh_last_error()
