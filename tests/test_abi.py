"""The C ABI on a host without a GPU: the library loads, exports every entry
point include/hh.h declares, sizes workspaces, and rejects bad arguments
before launching anything (fake, never-dereferenced device pointers)."""
import ctypes
import os
import re

import pytest

from hybrid_attention_ssm_amd import binding as hb
from hybrid_attention_ssm_amd.configs import CFG0_TINY, CFG1_SWA_8K, HYMBA_1P5B, TINY
from dataclasses import replace

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hh.h")
FAKE = 0x10000   # 16-byte aligned, never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[a-z_ ]+\**\s*\**(hh_[a-z_]+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["hh_prefill", "hh_decode_step", "hh_meta_prefix", "hh_prefill_workspace_size",
              "hh_decode_workspace_size", "hh_meta_prefix_workspace_size", "hh_last_error",
              "hh_version", "hh_prefill_workspace_layout", "hh_stage_attn", "hh_stage_ssm",
              "hh_stage_ssm_workspace_size"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    L = hb.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert "gfx950" in hb.hh_version()


def _weights(kv_producer=1):
    return hb.HHWeights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, kv_producer)


def _call_prefill(dims, B=1, n=64, window=16, ws_bytes=1 << 40, w=None, x=FAKE, meta=None, kv=None):
    d = hb.hh_dims(dims)
    w = w or _weights()
    meta = meta or hb.HHMeta(FAKE, FAKE, FAKE, FAKE)
    st = hb.HHSsmState(None, None)
    return hb.lib().hh_prefill(ctypes.byref(d), ctypes.byref(w), x, B, n, ctypes.byref(meta),
                               window, 0, FAKE, ctypes.byref(kv) if kv else None,
                               ctypes.byref(st), FAKE, ws_bytes, None)


def test_workspace_sizes():
    s1 = hb.hh_prefill_workspace_size(TINY, 1, 64)
    s2 = hb.hh_prefill_workspace_size(TINY, 2, 64)
    assert 0 < s1 < s2
    lay = hb.hh_prefill_workspace_layout(TINY, 1, 64)
    assert lay["total"] == s1
    offs = sorted(v for k, v in lay.items() if k != "total" and v is not None)
    assert offs == sorted(set(offs)) and all(o % 256 == 0 for o in offs)
    # consumer layers keep no K/V of their own
    lc = hb.hh_prefill_workspace_layout(TINY, 1, 64, kv_producer=False)
    assert lc["K"] is None and lc["V"] is None
    assert hb.hh_decode_workspace_size(HYMBA_1P5B, 128, 8192) > hb.hh_decode_workspace_size(HYMBA_1P5B, 128, 1024)
    assert hb.hh_prefill_workspace_size(replace(TINY, head_dim=48), 1, 64) == 0


@pytest.mark.parametrize("change,status", [
    (dict(head_dim=128), 2), (dict(d_state=8), 2), (dict(d_conv=5), 2), (dict(n_kv_heads=3), 1),
    (dict(d_model=60), 2), (dict(n_heads=0), 1), (dict(eps=-1.0), 1),
    (dict(rope_base=-10.0), 1), (dict(rope_base=0.5), 1), (dict(rope_base=float("nan")), 1),
    (dict(rope_base=float("inf")), 1), (dict(ssm_heads=-1), 1), (dict(ssm_heads=6), 1),
    (dict(ssm_heads=2), 1)])
def test_bad_dims_rejected(change, status):
    assert _call_prefill(replace(TINY, **change)) == status
    assert hb.hh_last_error() != ""


def test_bf16_needs_head_dim_64():
    assert _call_prefill(replace(TINY, dtype="bf16")) == 2
    assert "head_dim" in hb.hh_last_error()


def test_bad_arguments_rejected():
    assert _call_prefill(TINY, n=0) == 1
    assert _call_prefill(TINY, window=0) == 1
    assert _call_prefill(TINY, x=FAKE + 2) == 1                       # misaligned
    assert _call_prefill(TINY, w=hb.HHWeights(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1)) == 1
    # consumer without its producer's K/V
    assert _call_prefill(TINY, w=_weights(0)) == 1
    # ring cache smaller than the window
    kv = hb.HHKV(None, None, FAKE, FAKE, FAKE, 8, 1)
    assert _call_prefill(TINY, window=16, kv=kv) == 1
    assert "ring" in hb.hh_last_error()


def test_small_workspace_rejected():
    need = hb.hh_prefill_workspace_size(TINY, 1, 64)
    assert _call_prefill(TINY, ws_bytes=need - 1) == 3


def test_decode_validation():
    d = hb.hh_dims(TINY)
    w = _weights()
    meta = hb.HHMeta(FAKE, FAKE, FAKE, FAKE)
    st = hb.HHSsmState(FAKE, FAKE)
    kv = hb.HHKV(None, None, FAKE, FAKE, None, 16, 1)          # len missing
    r = hb.lib().hh_decode_step(ctypes.byref(d), ctypes.byref(w), FAKE, 4, ctypes.byref(meta),
                                16, 0, ctypes.byref(kv), ctypes.byref(st), FAKE, FAKE, 1 << 40, None)
    assert r == 1
    kv = hb.HHKV(None, None, FAKE, FAKE, FAKE, 16, 1)
    r = hb.lib().hh_decode_step(ctypes.byref(d), ctypes.byref(w), FAKE, 4, ctypes.byref(meta),
                                16, 1, ctypes.byref(kv), ctypes.byref(st), FAKE, FAKE, 1 << 40, None)
    assert r == 1 and "linear" in hb.hh_last_error()


def test_meta_prefix_validation():
    d = hb.hh_dims(replace(TINY, n_meta=0))
    w = _weights()
    r = hb.lib().hh_meta_prefix(ctypes.byref(d), ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE,
                                FAKE, 1 << 40, None)
    assert r == 1


def _block_weights(d_ff=96, norm=FAKE, kv_producer=1):
    return hb.HHBlockWeights(_weights(kv_producer), norm, norm, FAKE, FAKE, d_ff)


def _call_block_prefill(dims, bw, B=1, n=64, ws_bytes=1 << 40, x=FAKE, out=FAKE + 4096):
    d = hb.hh_dims(dims)
    meta = hb.HHMeta(FAKE, FAKE, FAKE, FAKE)
    st = hb.HHSsmState(None, None)
    return hb.lib().hh_block_prefill(ctypes.byref(d), ctypes.byref(bw), x, B, n, ctypes.byref(meta),
                                     16, 0, out, None, ctypes.byref(st), FAKE, ws_bytes, None)


def test_block_workspace_sizes():
    d = hb.hh_dims(TINY)
    L = hb.lib()
    layer = hb.hh_prefill_workspace_size(TINY, 1, 64)
    blk = L.hh_block_prefill_workspace_size(ctypes.byref(d), 96, 1, 64, 1)
    assert blk > layer
    assert L.hh_block_prefill_workspace_size(ctypes.byref(d), 98, 1, 64, 1) == 0   # d_ff % 4
    dec = L.hh_block_decode_workspace_size(ctypes.byref(d), 96, 4, 16, 1)
    assert dec > hb.hh_decode_workspace_size(TINY, 4, 16)
    assert L.hh_block_meta_prefix_workspace_size(ctypes.byref(d), 1) > hb.hh_meta_prefix_workspace_size(TINY)


def test_block_validation():
    assert _call_block_prefill(TINY, _block_weights(d_ff=6)) == 2
    assert "d_ff" in hb.hh_last_error()
    assert _call_block_prefill(TINY, _block_weights(norm=None)) == 1
    assert _call_block_prefill(TINY, _block_weights(), out=FAKE) == 1          # out aliases x
    assert "alias" in hb.hh_last_error()
    d = hb.hh_dims(TINY)
    need = hb.lib().hh_block_prefill_workspace_size(ctypes.byref(d), 96, 1, 64, 1)
    assert _call_block_prefill(TINY, _block_weights(), ws_bytes=need - 1) == 3


def test_linear_cache_shorter_than_prompt_rejected():
    """A producer's prefill into a linear cache must fit every prompt
    position (its length becomes len, where decode appends)."""
    kv = hb.HHKV(None, None, FAKE, FAKE, FAKE, 32, 0)           # linear, cap 32
    assert _call_prefill(TINY, n=64, kv=kv) == 1
    assert "linear cache" in hb.hh_last_error()
    kv = hb.HHKV(None, None, FAKE, FAKE, FAKE, 64, 0)           # cap == seqlen: accepted
    assert _call_prefill(TINY, n=64, kv=kv, ws_bytes=1) == 3    # (fails later, on the workspace)


@pytest.mark.parametrize("dims,status", [
    (replace(TINY, d_inner=8200), 2),                              # fp32 rows above 8192
    (replace(TINY, d_model=8200), 2),
    (replace(HYMBA_1P5B, d_inner=16448), 2),                       # bf16 rows above 16384
    (replace(TINY, d_inner=8192), 3)])                             # at the limit: accepted
def test_row_width_limits_checked_before_launch(dims, status):
    """The row kernels' width limits (decode norm merge, block pre-norms) are
    validated up front, so no call can fail after it has started updating
    the caller's state."""
    assert _call_prefill(dims, ws_bytes=1) == status
    if status == 2:
        assert "at most" in hb.hh_last_error()
    d = hb.hh_dims(dims)
    w = _weights()
    meta = hb.HHMeta(FAKE, FAKE, FAKE, FAKE)
    st = hb.HHSsmState(FAKE, FAKE)
    kv = hb.HHKV(None, None, FAKE, FAKE, FAKE, 16, 1)
    r = hb.lib().hh_decode_step(ctypes.byref(d), ctypes.byref(w), FAKE, 4, ctypes.byref(meta),
                                16, 0, ctypes.byref(kv), ctypes.byref(st), FAKE, FAKE, 1, None)
    assert r == status


def _call_decode(dims, B=4, ws_bytes=1 << 40):
    d = hb.hh_dims(dims)
    w = _weights()
    meta = hb.HHMeta(FAKE, FAKE, FAKE, FAKE)
    st = hb.HHSsmState(FAKE, FAKE)
    kv = hb.HHKV(None, None, FAKE, FAKE, FAKE, 16, 1)
    return hb.lib().hh_decode_step(ctypes.byref(d), ctypes.byref(w), FAKE, B, ctypes.byref(meta),
                                   16, 0, ctypes.byref(kv), ctypes.byref(st), FAKE, FAKE, ws_bytes, None)


@pytest.mark.parametrize("entry,stage", [("prefill", "inproj"), ("decode", "decode_inproj"),
                                         ("meta_prefix", "meta_inproj"), ("block_prefill", "block_norm1")])
def test_injected_launch_failure_surfaces_as_hip_error(entry, stage, monkeypatch):
    """HH_FAULT_INJECT=<stage> makes that stage's launch fail on the host,
    before anything is enqueued: the call returns HH_ERR_HIP naming the stage
    (here the first stage of each entry point, so no HIP call is made and the
    fake device pointers are never touched)."""
    monkeypatch.setenv("HH_FAULT_INJECT", stage)
    if entry == "prefill":
        r = _call_prefill(TINY)
    elif entry == "decode":
        r = _call_decode(TINY)
    elif entry == "meta_prefix":
        d, w = hb.hh_dims(TINY), _weights()
        r = hb.lib().hh_meta_prefix(ctypes.byref(d), ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE,
                                    FAKE, 1 << 40, None)
    else:
        r = _call_block_prefill(TINY, _block_weights())
    assert r == 4, r
    msg = hb.hh_last_error()
    assert "injected" in msg and stage in msg, msg
    # validation still comes first: a bad argument is reported as such
    assert _call_prefill(TINY, n=0) == 1


def test_stage_hooks_validate_before_launch():
    """The stage hooks reject bad arguments on the host (fake device pointers
    are never dereferenced)."""
    L = hb.lib()
    d = hb.hh_dims(TINY)
    ok = dict(q=FAKE, k=FAKE, v=FAKE, mk=FAKE, mv=FAKE, B=1, n=64, W=16, g=0, o=FAKE)

    def attn(**kw):
        a = dict(ok, **kw)
        return L.hh_stage_attn(ctypes.byref(d), a["q"], a["k"], a["v"], a["mk"], a["mv"], a["B"], a["n"],
                               a["W"], a["g"], a["o"], None)
    assert attn(q=None) == 1 and attn(o=FAKE + 4) == 1 and attn(mk=None) == 1
    assert attn(W=0) == 1 and attn(B=0) == 1 and attn(n=-1) == 1
    assert attn(W=0, g=1, mk=None, mv=None) == 1   # meta needed while n_meta > 0
    w = _weights()
    need = hb.hh_stage_ssm_workspace_size(TINY, 1, 64)
    assert need > 0

    def ssm(ws_bytes=need, xs=FAKE, z=FAKE, y=FAKE, wts=w):
        return L.hh_stage_ssm(ctypes.byref(d), ctypes.byref(wts), xs, z, FAKE, FAKE, None, None, 1, 64,
                              y, None, None, FAKE, ws_bytes, None)
    assert ssm(ws_bytes=need - 1) == 3
    assert ssm(xs=None) == 1 and ssm(z=None) == 1
    assert ssm(wts=hb.HHWeights(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1)) == 1   # no A
