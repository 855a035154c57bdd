#!/usr/bin/env python3
"""Benchmark of libhymba_hh on one MI355X.

Headline step: one hh_prefill of the Hymba-1.5B-shaped sliding-window
hybrid-head layer over 8192 tokens (batch 1, d_model 1600, 25/5 heads of 64,
128 meta tokens, window 1024, d_inner 3200, state 16, conv 4), bf16 storage
with fp32 accumulation, inputs already resident in HBM.  Reported beside it:
the batch-128 decode step (SWA producer + SWA consumer sharing one ring KV
cache + a global layer over 8192 cached positions).

Prints ONE JSON line.  Per-kernel durations come from HIP events recorded
by the library on the stream it launches on (hh_timing_*); the headline time
is a separate event-bracketed loop without those per-stage events.  After
both loops, --settle-steps more prefill steps run back to back and the second
half of them is timed: the rate once the GPU's clocks have settled under
continuous load, reported as "settled" beside (never as) the value.

  python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--only prefill|decode]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK = 2.5166e15   # dense bf16 FLOP/s, MI355X
HBM_PEAK = 8.0e12            # bytes/s, MI355X HBM3E
ROPE_BASE = 10000.0          # rotary base of the RoPE prefill line (the value does not change the work)
MAMBA2_HEADS = 64            # SSM heads of the Mamba2 prefill line (50 channels each)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the rocprofv3 counter
    summaries under profiles/ (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or
    None when there is none or the kernel's sources changed since."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "hbm_traffic_*.md"))):
        for line in open(path):
            if not line.startswith("traffic:"):
                continue
            kv = dict(tok.split("=", 1) for tok in line.split()[1:])
            if kv.get("kernel") != kernel or kv.get("workload") != workload:
                continue
            h = hashlib.sha256()
            for f in kv["sources"].split(","):
                with open(os.path.join(ROOT, f), "rb") as fh:
                    h.update(fh.read())
            if h.hexdigest()[:16] != kv["sha256"]:
                return None
            fb, wb = float(kv["fetch_bytes"]), float(kv["write_bytes"])
            return {"bytes": fb + wb, "fetch_bytes": fb, "write_bytes": wb,
                    "source": os.path.relpath(path, ROOT)}
    return None


# ---------------------------------------------------------------------------
# algorithmic work (what the method must do; masked-out attention pairs and
# padding are not counted)
# ---------------------------------------------------------------------------
def prefill_flops(dims, B, n, window, is_global, kv_producer=True):
    m = dims.n_meta
    T = B * n
    inproj = 2.0 * T * dims.d_model * dims.n_in(kv_producer)
    if is_global:
        real_pairs = n * (n + 1) // 2
    else:
        W = window
        real_pairs = sum(min(t + 1, W) for t in range(n)) if n <= 65536 else None
    pairs = B * (m * n + real_pairs)
    attention = 4.0 * dims.head_dim * dims.n_heads * pairs
    outproj = 2.0 * T * dims.fused_width * dims.d_model
    return dict(inproj=inproj, attention=attention, outproj=outproj,
                total=inproj + attention + outproj)


def decode_bytes(dims, B, layers, p, window, ring_cap, global_cap):
    """Algorithmic HBM bytes of one decode step over `layers` (list of
    (is_global, kv_producer)); p = position of the new token."""
    es = 2
    G, hd, m, D, N, k, d = (dims.n_kv_heads, dims.head_dim, dims.n_meta, dims.d_inner,
                            dims.d_state, dims.d_conv, dims.d_model)
    tot = 0.0
    attn = 0.0
    for is_global, prod in layers:
        w = dims.n_in(prod) * d * es + d * dims.fused_width * es
        small = 4 * (D + D * N + D * k + D + dims.attn_width + D)
        ssm = B * D * N * 4 * 2 + B * (k - 1) * D * 4 * 2
        io = B * d * es * 2
        keys = (p + 1) if is_global else min(window, p + 1)
        kv_read = B * G * keys * hd * es * 2 + G * m * hd * es * 2
        append = B * G * hd * es * 2 if prod else 0
        tot += w + small + ssm + io + kv_read + append
        attn += kv_read
    return tot, attn


# ---------------------------------------------------------------------------
def bench_prefill(args, hb, torch, rope_base=0.0, ssm_heads=0, concurrent=False, settle_steps=0,
                  one_launch=False):
    """The 8k SWA prefill; rope_base > 0 times the same layer with Q and K
    turned by the rotary embedding (same inputs), ssm_heads > 0 with Mamba2
    SSM heads (inputs drawn for that layout); concurrent runs the SSM branch
    on the library's side stream (HH_CONCURRENT_BRANCHES=1); one_launch runs
    the attention and scan pass 3 in one grid (HH_ONE_LAUNCH_BRANCHES=1)."""
    from dataclasses import replace
    from hybrid_attention_ssm_amd.configs import CFG1_SWA_8K
    from hybrid_attention_ssm_amd.synth import prefill_inputs
    w = CFG1_SWA_8K
    dims = replace(w.dims, rope_base=rope_base, ssm_heads=ssm_heads)
    w = replace(w, dims=dims)
    B, n, W = w.batch, w.seqlen, w.window
    tag = ((f" (RoPE base {rope_base:g})" if rope_base else "") +
           (f" (Mamba2 heads: {ssm_heads})" if ssm_heads else "") +
           (" (branches on two streams)" if concurrent else "") +
           (" (attention and scan pass 3 in one launch)" if one_launch else ""))
    prev_env = {k: os.environ.get(k) for k in ("HH_CONCURRENT_BRANCHES", "HH_ONE_LAUNCH_BRANCHES")}
    os.environ["HH_CONCURRENT_BRANCHES"] = "1" if concurrent else "0"
    os.environ["HH_ONE_LAUNCH_BRANCHES"] = "1" if one_launch else "0"
    log(f"[bench] prefill setup {w.name}{tag}")
    inp = prefill_inputs(w)
    sd = hb.storage_dtype(dims)
    dev = "cuda"
    layer = hb.upload_weights(dims, inp["weights"])
    meta = hb.hh_meta_prefix(layer, hb.to_device(inp["R"], sd))
    x = hb.to_device(inp["x"], sd)
    G, hd, D, N, k = dims.n_kv_heads, dims.head_dim, dims.d_inner, dims.d_state, dims.d_conv
    out = torch.empty(B, n, dims.d_model, dtype=sd, device=dev)
    full_k = torch.empty(B, G, n, hd, dtype=sd, device=dev)
    full_v = torch.empty_like(full_k)
    ck = torch.zeros(B, G, W, hd, dtype=sd, device=dev)
    cv = torch.zeros_like(ck)
    length = torch.zeros(B, dtype=torch.int32, device=dev)
    h = torch.empty(B, D, N, dtype=torch.float32, device=dev)
    conv = torch.empty(B, k - 1, D, dtype=torch.float32, device=dev)
    ws = torch.empty(hb.hh_prefill_workspace_size(dims, B, n), dtype=torch.uint8, device=dev)
    kv = hb.make_kv(full_k, full_v, ck, cv, length, W, True)
    ms = hb.make_meta(meta["k"], meta["v"], meta["h0"], meta["conv_tail"])

    def step():
        hb.hh_prefill(layer, x, ms, W, False, out, kv=kv, state_h=h, state_conv=conv, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(args.steps):
        step()
    s1.record()
    torch.cuda.synchronize()
    ms_step = s0.elapsed_time(s1) / args.steps
    # per-stage event timing over another K steps
    hb.hh_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    stages = hb.hh_timing_read()
    hb.hh_timing_enable(False)
    settled = None
    if settle_steps > 0:
        # the rate once the GPU's clocks have settled under continuous load
        # (reported beside the timed steps, never as the value): settle_steps
        # more steps back to back, the second half of them timed
        for _ in range(settle_steps // 2):
            step()
        s2, s3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s2.record()
        for _ in range(settle_steps - settle_steps // 2):
            step()
        s3.record()
        torch.cuda.synchronize()
        settled = s2.elapsed_time(s3) / (settle_steps - settle_steps // 2)
    for k, v in prev_env.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v
    fl = prefill_flops(dims, B, n, W, False)
    st_ms = {name: tot / cnt for name, (cnt, tot) in stages.items()}
    log(f"[bench] prefill{tag} {ms_step:.3f} ms/step; stages " +
        ", ".join(f"{k}={v * 1e3:.1f}us" for k, v in st_ms.items()))
    return dict(workload=w.name, dims=dims, B=B, n=n, W=W, ms_step=ms_step, settled_ms=settled,
                settle_steps=settle_steps, stages=st_ms,
                flops=fl, inp=inp)


def bench_decode(args, hb, torch):
    from hybrid_attention_ssm_amd.configs import CFG3_DECODE
    from hybrid_attention_ssm_amd.synth import decode_inputs
    w = CFG3_DECODE
    dims = w.dims
    B, W = w.batch, w.window
    log(f"[bench] decode setup {w.name}")
    inp = decode_inputs(w)
    sd = hb.storage_dtype(dims)
    dev = "cuda"
    slack = args.warmup + 2 * args.steps + 2
    caches = {}
    for name, c in inp["caches"].items():
        cap = c["cap"] if c["is_ring"] else c["cap"] + slack   # the linear cache grows one per step
        kk = torch.zeros(B, dims.n_kv_heads, cap, dims.head_dim, dtype=sd, device=dev)
        vv = torch.zeros_like(kk)
        kk[:, :, :c["cap"]] = hb.to_device(c["k"], sd)
        vv[:, :, :c["cap"]] = hb.to_device(c["v"], sd)
        ln = hb.to_device(c["len"], torch.int32)
        caches[name] = dict(k=kk, v=vv, len=ln, cap=cap, is_ring=c["is_ring"],
                            mk=hb.to_device(c["meta_k"], sd), mv=hb.to_device(c["meta_v"], sd))
        caches[name]["kv"] = hb.make_kv(None, None, kk, vv, ln, cap, c["is_ring"])
        caches[name]["meta"] = hb.make_meta(caches[name]["mk"], caches[name]["mv"], None, None)
    layers = []
    for lay in inp["layers"]:
        spec = lay["spec"]
        layers.append(dict(
            spec=spec, layer=hb.upload_weights(dims, lay["weights"]),
            h=hb.to_device(lay["h"], torch.float32), conv=hb.to_device(lay["conv"], torch.float32),
            x=hb.to_device(lay["x_t"], sd),
            out=torch.empty(B, dims.d_model, dtype=sd, device=dev)))
    wsz = max(hb.hh_decode_workspace_size(dims, B, caches[L["spec"].cache]["cap"],
                                          L["spec"].kv_producer) for L in layers)
    ws = torch.empty(wsz, dtype=torch.uint8, device=dev)

    def step():
        for L in layers:
            c = caches[L["spec"].cache]
            hb.hh_decode_step(L["layer"], L["x"], c["meta"], W, L["spec"].is_global, c["kv"],
                              L["h"], L["conv"], L["out"], ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    p_first = int(caches["global"]["len"][0].item())
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(args.steps):
        step()
    s1.record()
    torch.cuda.synchronize()
    ms_step = s0.elapsed_time(s1) / args.steps
    hb.hh_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    stages = hb.hh_timing_read()
    hb.hh_timing_enable(False)
    specs = [(L["spec"].is_global, L["spec"].kv_producer) for L in layers]
    p_mid = p_first + args.steps // 2          # mean position over the timed steps
    tot_bytes, attn_bytes = decode_bytes(dims, B, specs, p_mid, W, W, w.global_cap)
    # the stage loop ran at positions p_first + steps .. p_first + 2 steps - 1
    _, attn_bytes_stage = decode_bytes(dims, B, specs, p_first + args.steps + args.steps // 2,
                                       W, W, w.global_cap)
    # the global layer's K/V bytes per launch at the stage loop's mean position
    p_stage = p_first + args.steps + args.steps // 2
    G, hd, m = dims.n_kv_heads, dims.head_dim, dims.n_meta
    global_attn_bytes = B * G * (p_stage + 1) * hd * 2 * 2 + G * m * hd * 2 * 2
    st = {name: (cnt, tot) for name, (cnt, tot) in stages.items()}
    log(f"[bench] decode {ms_step:.3f} ms/step; stages " +
        ", ".join(f"{k}={v[1] / v[0] * 1e3:.1f}us x{v[0]}" for k, v in st.items()))
    return dict(workload=w.name, B=B, ms_step=ms_step, stages=st, bytes=tot_bytes,
                attn_bytes_step=attn_bytes_stage, global_attn_bytes=global_attn_bytes, inp=inp,
                context=p_first)


def bench_stack(args, hb, torch):
    """One decode step through the 32 blocks of the 1.5B stack (layer, pre-norms,
    residuals, MLP), batch 128 at context 8191+.  Weights, caches, meta K/V
    and states are normal draws made on the device (seeded torch generator):
    this line measures speed only; the block's parity is tested elsewhere."""
    from hybrid_attention_ssm_amd.configs import STACK_DECODE
    w = STACK_DECODE
    dims, B, W = w.dims, w.batch, w.window
    sd = hb.storage_dtype(dims)
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    d, D, N, k = dims.d_model, dims.d_inner, dims.d_state, dims.d_conv
    G, hd, m, d_ff = dims.n_kv_heads, dims.head_dim, dims.n_meta, w.d_ff
    f32 = torch.float32

    def normal(shape, std=1.0, dtype=sd):
        t = torch.randn(shape, generator=gen, device=dev, dtype=f32)
        if std != 1.0:
            t.mul_(std)
        return t.to(dtype).contiguous()

    steps = max(4, args.steps // 2)
    slack = args.warmup + steps + 2
    plan = w.layer_plan()
    log(f"[bench] stack setup {w.name} ({len(plan)} blocks)")
    caches = {}
    for is_g, prod, name in plan:
        if name in caches:
            continue
        cap = w.global_cap + slack if is_g else W
        kk, vv = normal((B, G, cap, hd)), normal((B, G, cap, hd))
        ln = torch.full((B,), w.context, dtype=torch.int32, device=dev)
        mk, mv = normal((G, m, hd)), normal((G, m, hd))
        caches[name] = dict(t=(kk, vv, ln, mk, mv), kv=hb.make_kv(None, None, kk, vv, ln, cap, not is_g),
                            meta=hb.make_meta(mk, mv, None, None), cap=cap)
    blocks = []
    for is_g, prod, name in plan:
        t = {"w_in": normal((dims.n_in(prod), d), (1.0 / d) ** 0.5),
             "dt_bias": torch.full((D,), -4.0, dtype=f32, device=dev),
             "A": -torch.rand((D, N), generator=gen, device=dev, dtype=f32).mul_(15.0).add_(1.0),
             "conv_w": normal((D, k), (1.0 / k) ** 0.5, f32), "conv_b": torch.zeros(D, dtype=f32, device=dev),
             "beta_attn": torch.ones(dims.attn_width, dtype=f32, device=dev),
             "beta_ssm": torch.ones(D, dtype=f32, device=dev),
             "w_out": normal((d, dims.fused_width), (1.0 / dims.fused_width) ** 0.5),
             "norm1": torch.ones(d, dtype=f32, device=dev), "norm2": torch.ones(d, dtype=f32, device=dev),
             "w_gate_up": normal((2 * d_ff, d), (1.0 / d) ** 0.5), "w_down": normal((d, d_ff), (1.0 / d_ff) ** 0.5),
             "h": normal((B, D, N), 1.0, f32), "conv": normal((B, k - 1, D), 1.0, f32)}
        P = hb._ptr
        ws_ = hb.HHWeights(P(t["w_in"]), P(t["dt_bias"]), P(t["A"]), P(t["conv_w"]), P(t["conv_b"]),
                           P(t["beta_attn"]), P(t["beta_ssm"]), P(t["w_out"]), 1 if prod else 0)
        bs = hb.HHBlockWeights(ws_, P(t["norm1"]), P(t["norm2"]), P(t["w_gate_up"]), P(t["w_down"]), d_ff)
        blk = hb.DeviceBlock(dims, hb.DeviceLayer(dims, t, ws_), t, bs)
        blocks.append(dict(block=blk, is_global=is_g, cache=caches[name]))
    wsz = max(hb.hh_block_decode_workspace_size(b["block"], B, b["cache"]["cap"]) for b in blocks)
    ws = torch.empty(wsz, dtype=torch.uint8, device=dev)
    xa, xb = normal((B, d)), torch.empty(B, d, dtype=sd, device=dev)

    def step():
        cur, nxt = xa, xb
        for b in blocks:
            c = b["cache"]
            hb.hh_block_decode_step(b["block"], cur, c["meta"], W, b["is_global"], c["kv"],
                                    b["block"].tensors["h"], b["block"].tensors["conv"], nxt, ws=ws)
            cur, nxt = nxt, cur

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(steps):
        step()
    s1.record()
    torch.cuda.synchronize()
    ms_step = s0.elapsed_time(s1) / steps
    p_mid = w.context + 2 + steps // 2
    layers = [(g_, p_) for g_, p_, _ in plan]
    mixer_bytes, _ = decode_bytes(dims, B, layers, p_mid, W, W, w.global_cap)
    mlp_bytes = len(plan) * (3 * d * d_ff * 2 + 2 * d * 4 + B * d * 2 * 2)
    tot = mixer_bytes + mlp_bytes
    log(f"[bench] stack {ms_step:.3f} ms/step ({B / (ms_step * 1e-3):.0f} tok/s)")
    return {"workload": f"{w.name}: {len(plan)} Hymba-1.5B-shaped blocks (full attention in blocks "
                        f"{', '.join(map(str, w.global_layers))}; sliding-window blocks in KV-sharing pairs; "
                        f"MLP {d_ff}), batch {B}, context {w.context}+",
            "value": B / (ms_step * 1e-3), "unit": "tok/s", "ms_per_step": ms_step, "steps": steps,
            "algorithmic_bytes_per_step": tot, "hbm_frac_step": tot / (ms_step * 1e-3) / HBM_PEAK,
            "data": "synthetic, drawn on the device"}


# ---------------------------------------------------------------------------
def cpu_baseline(pre, dec, args):
    """The CPU oracle (as it stands) on a bounded sample of each workload."""
    import numpy as np
    from oracle import hymba_ref as ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    res = {}
    if pre is not None:
        inp = pre["inp"]
        ns = args.cpu_sample_tokens
        dims = pre["dims"]
        t0 = time.perf_counter()
        ref.prefill(dims.as_dict(), inp["weights"], inp["R"], inp["x"][:, :ns], pre["W"], False)
        dt = time.perf_counter() - t0
        res["prefill"] = dict(value=ns / dt, seconds=dt,
                              sample=f"oracle prefill of {ns} of the 8192 tokens "
                                     f"(same layer, meta rows included), fp64")
    if dec is not None:
        from hybrid_attention_ssm_amd.configs import CFG3_DECODE
        w = CFG3_DECODE
        inp = dec["inp"]
        S = np.arange(args.cpu_sample_seqs)
        t0 = time.perf_counter()
        caches = {name: dict(k=c["k"][S], v=c["v"][S], len=c["len"][S], is_ring=c["is_ring"])
                  for name, c in inp["caches"].items()}
        for lay in inp["layers"]:
            spec = lay["spec"]
            c = inp["caches"][spec.cache]
            r = ref.decode_step(w.dims.as_dict(), lay["weights"], lay["x_t"][S], c["meta_k"],
                                c["meta_v"], w.window, spec.is_global, caches[spec.cache],
                                lay["h"][S], lay["conv"][S])
            if spec.kv_producer:
                caches[spec.cache] = dict(k=r["cache_k"], v=r["cache_v"], len=r["len"],
                                          is_ring=c["is_ring"])
        dt = time.perf_counter() - t0
        res["decode"] = dict(value=len(S) / dt, seconds=dt,
                             sample=f"oracle decode step (3 layers) for {len(S)} of the 128 "
                                    f"sequences, fp64")
    res["cores"] = threads
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    res["cpu"] = cpu
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-steps", type=int, default=160,
                    help="extra 8k prefill steps after the timed ones, the second half timed "
                         "(the settled rate, reported beside the value; 0 = skip)")
    ap.add_argument("--only", choices=["prefill", "decode", "both"], default="both")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the 32-block decode stack line")
    ap.add_argument("--no-rope", action="store_true",
                    help="skip the prefill line with the rotary embedding of Q and K")
    ap.add_argument("--no-mamba2", action="store_true",
                    help="skip the prefill line with Mamba2 SSM heads")
    ap.add_argument("--no-branches", action="store_true",
                    help="skip the prefill lines with the SSM branch on a second stream and with the "
                         "attention and scan pass 3 in one launch")
    ap.add_argument("--cpu-sample-tokens", type=int, default=8192,
                    help="prefill tokens the CPU oracle runs (default: the whole 8k workload)")
    ap.add_argument("--cpu-sample-seqs", type=int, default=64,
                    help="decode sequences the CPU oracle steps (of 128)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB (the known-size kernel "
                         "that scales the HBM byte counters) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build measures one GPU only (--gpus {args.gpus}, WORLD_SIZE "
              f"{world} requested); the layer's multi-GPU sharding is a design note, not built.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from hybrid_attention_ssm_amd import binding as hb
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    hb.lib()
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {n} bytes x5 (each launch reads {n} and writes {n} bytes)")
        return

    pre = (bench_prefill(args, hb, torch, settle_steps=args.settle_steps)
           if args.only in ("prefill", "both") else None)
    pre_rope = pre_m2 = None
    if pre is not None and not args.no_rope:
        pre_rope = bench_prefill(args, hb, torch, rope_base=ROPE_BASE)
    if pre is not None and not args.no_mamba2:
        pre_m2 = bench_prefill(args, hb, torch, ssm_heads=MAMBA2_HEADS)
    pre_br = pre_ol = None
    if pre is not None and not args.no_branches:
        pre_br = bench_prefill(args, hb, torch, concurrent=True)
        pre_ol = bench_prefill(args, hb, torch, one_launch=True)
    dec = bench_decode(args, hb, torch) if args.only in ("decode", "both") else None
    stack = None
    if args.only in ("decode", "both") and not args.no_stack:
        try:
            stack = bench_stack(args, hb, torch)
        except Exception as exc:   # the stack line is extra: report it, keep the main line
            log(f"[bench] stack failed: {exc!r}")
            stack = {"error": repr(exc)}

    rec = {"metric": "hybrid-head layer prefill tok/s @8k + decode tok/s @B128; % of MFMA/HBM peak",
           "higher_is_better": True, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "unit": "tok/s"}
    if pre is not None:
        fl = pre["flops"]
        toks = pre["B"] * pre["n"] / (pre["ms_step"] * 1e-3)
        t_in = pre["stages"].get("inproj")
        rec.update(value=toks, ms_per_step=pre["ms_step"])
        rec["config"] = {"workload": f"{pre['workload']}: Hymba-1.5B-shaped SWA hybrid-head "
                                     f"layer prefill (d 1600, 25/5 heads x 64, 128 meta, W 1024, "
                                     f"d_inner 3200, N 16, conv 4)",
                         "global_batch": pre["B"], "seq_len": pre["n"], "parallelism": "none"}
        rec["mfma_frac_layer"] = fl["total"] / (pre["ms_step"] * 1e-3) / MFMA_BF16_PEAK
        if pre["settled_ms"]:
            # the GPU's clocks ramp over the first ~30 ms of continuous load: the
            # timed steps above run partly inside that ramp
            rec["settled"] = {"ms_per_step": pre["settled_ms"],
                              "tok_per_s": pre["B"] * pre["n"] / (pre["settled_ms"] * 1e-3),
                              "mfma_frac_layer": fl["total"] / (pre["settled_ms"] * 1e-3) / MFMA_BF16_PEAK,
                              "steps": pre["settle_steps"] - pre["settle_steps"] // 2,
                              "after_steps": pre["settle_steps"] // 2,
                              "note": "continuous prefill steps after the timed and stage-timed ones; "
                                      "not the value"}
        rec["algorithmic_gflop_per_step"] = fl["total"] / 1e9
        rec["stage_us"] = {k: v * 1e3 for k, v in pre["stages"].items()}
        t_scan = pre["stages"].get("scan")
        if t_scan:
            # the scan step alone: xs, Delta (fp32), z (bf16) and B|C (fp32) read, Y (bf16) written,
            # and one exp per (token, channel, state) of the recurrence
            dd = pre["dims"]
            T = pre["B"] * pre["n"]
            sb = T * dd.d_inner * (4 + 4 + 2 + 2) + T * 2 * dd.d_state * 4
            ex = T * dd.d_inner * dd.d_state
            rec["scan"] = {"us": t_scan * 1e3, "algorithmic_bytes": sb,
                           "GB_per_s": sb / (t_scan * 1e-3) / 1e9, "frac_hbm": sb / (t_scan * 1e-3) / HBM_PEAK,
                           "recurrence_exps": ex, "exps_per_s": ex / (t_scan * 1e-3)}
        if pre_rope is not None:
            # the same workload with RoPE on Q and K (turned in the in-projection's epilogue)
            t_in_r = pre_rope["stages"].get("inproj")
            rec["rope"] = {"rope_base": ROPE_BASE, "ms_per_step": pre_rope["ms_step"],
                           "value": pre["B"] * pre["n"] / (pre_rope["ms_step"] * 1e-3), "unit": "tok/s",
                           "mfma_frac_layer": fl["total"] / (pre_rope["ms_step"] * 1e-3) / MFMA_BF16_PEAK,
                           "stage_us": {k: v * 1e3 for k, v in pre_rope["stages"].items()},
                           "inproj_extra_us": (t_in_r - t_in) * 1e3 if (t_in_r and t_in) else None}
        if pre_m2 is not None:
            # the same workload with Mamba2 SSM heads: the dt block shrinks to one column per head
            # and the scan takes one exp per (token, channel)
            dd = pre_m2["dims"]
            T = pre["B"] * pre["n"]
            fl2 = pre_m2["flops"]
            t_scan2 = pre_m2["stages"].get("scan")
            rec["mamba2"] = {"ssm_heads": MAMBA2_HEADS, "ms_per_step": pre_m2["ms_step"],
                             "value": T / (pre_m2["ms_step"] * 1e-3), "unit": "tok/s",
                             "mfma_frac_layer": fl2["total"] / (pre_m2["ms_step"] * 1e-3) / MFMA_BF16_PEAK,
                             "algorithmic_gflop_per_step": fl2["total"] / 1e9,
                             "stage_us": {k: v * 1e3 for k, v in pre_m2["stages"].items()},
                             "scan_exps": T * dd.d_inner,
                             "scan_exps_per_s": T * dd.d_inner / (t_scan2 * 1e-3) if t_scan2 else None}
        if pre_br is not None:
            # the same workload with the SSM branch on the library's side stream (opt-in: measured
            # slower than one stream); stage times overlap there, so only the step time is reported
            rec["branches"] = {"mode": "HH_CONCURRENT_BRANCHES=1 (input projection in two row ranges, "
                                       "scan summaries beside the second, rest of the scan beside the attention)",
                               "ms_per_step": pre_br["ms_step"],
                               "value": pre["B"] * pre["n"] / (pre_br["ms_step"] * 1e-3), "unit": "tok/s",
                               "vs_one_stream": pre["ms_step"] / pre_br["ms_step"]}
        if pre_ol is not None:
            # the attention and scan pass 3 in one grid (opt-in: measured slower than two launches)
            rec["one_launch"] = {"mode": "HH_ONE_LAUNCH_BRANCHES=1 (scan passes 1 and 2, then one grid of "
                                         "attention and scan pass-3 workgroups)",
                                 "ms_per_step": pre_ol["ms_step"],
                                 "value": pre["B"] * pre["n"] / (pre_ol["ms_step"] * 1e-3), "unit": "tok/s",
                                 "vs_two_launches": pre["ms_step"] / pre_ol["ms_step"],
                                 "stage_us": {k: v * 1e3 for k, v in pre_ol["stages"].items()}}
        if t_in:
            ach = fl["inproj"] / (t_in * 1e-3)
            tr = measured_traffic("gemm_bf16_lds", pre["workload"])
            rec["roofline"] = {"kernel": "in-proj GEMM (gemm_bf16_lds, InProjEpi)", "bound": "mfma",
                               "achieved": ach / 1e12, "peak": MFMA_BF16_PEAK / 1e12,
                               "unit": "TFLOP/s", "frac": ach / MFMA_BF16_PEAK,
                               "traffic": tr["bytes"] if tr else None,
                               "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE)",
                               "traffic_detail": tr,
                               "flop_per_launch": fl["inproj"], "avg_launch_us": t_in * 1e3}
    if dec is not None:
        B = dec["B"]
        st = dec["stages"]
        d = {"workload": f"{dec['workload']}: 3 layers per step (SWA producer + SWA consumer "
                         f"sharing a 1024-slot ring cache, global layer over the full cache), "
                         f"context {dec['context']}+",
             "value": B / (dec["ms_step"] * 1e-3), "unit": "tok/s", "ms_per_step": dec["ms_step"],
             "hbm_frac_step": dec["bytes"] / (dec["ms_step"] * 1e-3) / HBM_PEAK,
             "algorithmic_bytes_per_step": dec["bytes"],
             # the same fraction over the 2.01 GB per step of the design notes' count (without
             # the fp32 conv-history bytes)
             "hbm_frac_step_2p01GB": 2.01e9 / (dec["ms_step"] * 1e-3) / HBM_PEAK,
             "stage_us": {k: v[1] / v[0] * 1e3 for k, v in st.items()}}
        if "decode_attention_global" in st:
            cnt, tot = st["decode_attention_global"]
            ach = dec["global_attn_bytes"] / (tot / cnt * 1e-3)
            tr = measured_traffic("decode_attn_dma", dec["workload"])
            d["roofline"] = {"kernel": "decode attention of the global layer (decode_attn_dma; "
                                       "its split partials are merged by the decode norm kernel)",
                             "bound": "hbm", "achieved": ach / 1e9, "peak": HBM_PEAK / 1e9,
                             "unit": "GB/s", "frac": ach / HBM_PEAK,
                             "traffic": tr["bytes"] if tr else None,
                             "traffic_unit": "HBM bytes per launch of decode_attn_dma "
                                             "(FETCH_SIZE + WRITE_SIZE)",
                             "traffic_detail": tr,
                             "bytes_per_launch": dec["global_attn_bytes"],
                             "avg_launch_us": tot / cnt * 1e3}
        rec["decode"] = d
        if pre is None:
            rec.update(value=d["value"], ms_per_step=d["ms_per_step"],
                       config={"workload": d["workload"], "global_batch": B, "seq_len": 1,
                               "parallelism": "none"})
    if stack is not None:
        rec["stack"] = stack
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        cb = cpu_baseline(pre, dec, args)
        main_key = "prefill" if pre is not None else "decode"
        rec["cpu_baseline"] = {"value": cb[main_key]["value"], "unit": "tok/s", "cores": cb["cores"],
                               "kind": "oracle", "sample": cb[main_key]["sample"],
                               "seconds": cb[main_key]["seconds"], "cpu": cb["cpu"],
                               "threads": "cores = the BLAS thread count, used by the oracle's matrix "
                                          "products (the projections); its per-query attention loop "
                                          "and the sequential recurrence run on one thread"}
        if pre is not None and "decode" in cb:
            rec["cpu_baseline"]["decode"] = cb["decode"]
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
