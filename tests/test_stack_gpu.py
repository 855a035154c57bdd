"""GPU parity of decode steps through a stack of blocks (the architecture
figure's stack: full-attention blocks first, in the middle and last; the
sliding-window blocks between them in KV-sharing pairs, a leftover one
producing for itself; meta K/V per cache; each block's own SSM state).

Six blocks with full attention in blocks 0, 3 and 5: block 1 produces into a
ring that block 2 reads, block 4 produces alone.  Batch 4, caches holding 20
positions (the 16-slot rings have wrapped), three steps.

* Stack output: the oracle chains block_decode_step through the same plan
  on its own values; compared after every step with the GPU's output.  fp32:
  bar 1e-4.  bf16: the path stores every activation it hands between kernels
  (inside a block and from block to block) in bf16, which moves the result by
  itself; the bar is the layer's 3e-2 plus that effect, measured as the
  distance between the exact chain and the same chain on stored values (the
  oracle's `store` map plus the rounding of each block's output).
* Every block's SSM state and conv history and every cache's slots and
  lengths after the last step: against the oracle chain fed, block by block
  and step by step, the inputs the GPU's blocks received (on stored values
  for bf16), so each block's state is checked on its own inputs, at the
  layer's bar; slots no step wrote keep their bits.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from hybrid_attention_ssm_amd import binding as hb
from hybrid_attention_ssm_amd.configs import MLP_HIDDEN_TINY, TINY, StackWorkload
from hybrid_attention_ssm_amd.synth import round_bf16, stack_inputs
from oracle import hymba_ref as ref
from tests.harness import TOL, np_of, rel_err
from tests.test_decode_gpu import SMALL_BF16

pytestmark = pytest.mark.gpu

STEPS = 3
TINY_STACK = StackWorkload("stack6_tiny", 80, TINY, MLP_HIDDEN_TINY, batch=4, context=20, window=16,
                           global_cap=32, n_layers=6, global_layers=(0, 3, 5))
SMALL_STACK = replace(TINY_STACK, name="stack6_small_bf16", seed=81, dims=SMALL_BF16, d_ff=256)


def _oracle_chain(w, inp, store, forced=None):
    """Stack outputs per step and the final states/caches, oracle side.
    forced[s][i]: the input block i received at step s (teacher forcing);
    None: each block reads the previous block's oracle output (rounded by
    `store` when given)."""
    dims = w.dims
    caches = {n: dict(k=c["k"].astype(np.float64), v=c["v"].astype(np.float64), len=c["len"].copy(),
                      is_ring=c["is_ring"]) for n, c in inp["caches"].items()}
    states = [(b["h"].astype(np.float64), b["conv"].astype(np.float64)) for b in inp["blocks"]]
    outs = []
    for s in range(STEPS):
        cur = inp["x"][s].astype(np.float64)
        for i, blk in enumerate(inp["blocks"]):
            if forced is not None:
                cur = forced[s][i]
            c = inp["caches"][blk["cache"]]
            kw = {} if store is None else dict(store=store)
            r = ref.block_decode_step(dims.as_dict(), blk["weights"], cur, c["meta_k"], c["meta_v"],
                                      w.window, blk["is_global"], caches[blk["cache"]], states[i][0],
                                      states[i][1], **kw)
            if blk["kv_producer"]:
                caches[blk["cache"]] = dict(k=r["cache_k"], v=r["cache_v"], len=r["len"],
                                            is_ring=c["is_ring"])
            states[i] = (r["h"], r["conv"])
            cur = r["out"] if store is None else store(r["out"]).astype(np.float64)
        outs.append(cur)
    return outs, states, caches


@pytest.mark.parametrize("w", [TINY_STACK, SMALL_STACK], ids=lambda w: w.name)
def test_decode_stack_matches_oracle_chain(w):
    dims = w.dims
    print(f"case {w.name}: {w.n_layers} blocks, plan {w.layer_plan()}", flush=True)
    inp = stack_inputs(w, STEPS, varied=True)
    sd = hb.storage_dtype(dims)
    B, d = w.batch, dims.d_model
    dev = {}
    for name, c in inp["caches"].items():
        kk, vv = hb.to_device(c["k"], sd), hb.to_device(c["v"], sd)
        ln = hb.to_device(c["len"], torch.int32)
        mk, mv = hb.to_device(c["meta_k"], sd), hb.to_device(c["meta_v"], sd)
        dev[name] = dict(k=kk, v=vv, len=ln, mk=mk, mv=mv,
                         kv=hb.make_kv(None, None, kk, vv, ln, c["cap"], c["is_ring"]),
                         meta=hb.make_meta(mk, mv, None, None))
    blocks = []
    for blk in inp["blocks"]:
        blocks.append(dict(dev=hb.upload_block_weights(dims, blk["weights"]),
                           h=hb.to_device(blk["h"], torch.float32),
                           conv=hb.to_device(blk["conv"], torch.float32)))
    outs, inputs = [], []
    for s in range(STEPS):
        cur = hb.to_device(inp["x"][s], sd)
        inputs.append([])
        for blk, b in zip(inp["blocks"], blocks):
            c = dev[blk["cache"]]
            inputs[-1].append(cur)
            nxt = torch.empty(B, d, dtype=sd, device="cuda")
            hb.hh_block_decode_step(b["dev"], cur, c["meta"], w.window, blk["is_global"], c["kv"],
                                    b["h"], b["conv"], nxt)
            cur = nxt
        torch.cuda.synchronize()
        outs.append(np_of(cur))
    forced = [[np_of(t) for t in step] for step in inputs]

    tol = TOL[dims.dtype]
    store = round_bf16 if dims.dtype == "bf16" else None
    exact_outs = _oracle_chain(w, inp, None)[0]
    stored_outs = _oracle_chain(w, inp, store)[0] if store is not None else exact_outs
    _, want_states, want_caches = _oracle_chain(w, inp, store, forced=forced)
    for s in range(STEPS):
        e = rel_err(outs[s], exact_outs[s])
        e_store = rel_err(stored_outs[s], exact_outs[s])
        print(f"  step {s}: out err {e:.2e} (bar {tol:.0e} + storage effect {e_store:.2e}; "
              f"vs stored-value chain {rel_err(outs[s], stored_outs[s]):.2e})", flush=True)
        assert e <= tol + e_store
    for i, (blk, b) in enumerate(zip(inp["blocks"], blocks)):
        e_h = rel_err(np_of(b["h"]), want_states[i][0])
        e_c = rel_err(np_of(b["conv"]), want_states[i][1])
        print(f"  block {i} ({blk['cache']}, global={blk['is_global']}, producer={blk['kv_producer']}) "
              f"h={e_h:.2e} conv={e_c:.2e}", flush=True)
        assert e_h <= tol and e_c <= tol
    for name, c in dev.items():
        o = want_caches[name]
        e_k, e_v = rel_err(np_of(c["k"]), o["k"]), rel_err(np_of(c["v"]), o["v"])
        print(f"  cache {name}: k={e_k:.2e} v={e_v:.2e} len={c['len'].cpu().numpy()}", flush=True)
        assert e_k <= tol and e_v <= tol
        assert np.array_equal(c["len"].cpu().numpy(), o["len"])
        # slots no step wrote keep their bits
        cap = inp["caches"][name]["cap"]
        written = {(p % cap if inp["caches"][name]["is_ring"] else p)
                   for p in range(w.context, w.context + STEPS)}
        keep = [j for j in range(cap) if j not in written]
        src = inp["caches"][name]
        assert np.array_equal(np_of(c["k"])[:, :, keep], src["k"][:, :, keep].astype(np.float64))
        assert np.array_equal(np_of(c["v"])[:, :, keep], src["v"][:, :, keep].astype(np.float64))
