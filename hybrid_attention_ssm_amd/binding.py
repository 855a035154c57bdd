"""ctypes binding of libhymba_hh (include/hh.h): argument marshalling only.

Every step of the layer runs in the HIP library; torch supplies device memory
and the current stream.  The functions carry the C names.  Importing this
module does not need a GPU; calling into the library does, and a missing
library raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import LayerDims

# HH_LIB_PATH selects another build of the same library (the host-sanitizer
# build of the ABI check); there is no other implementation to fall back to
LIB_PATH = os.environ.get("HH_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                         "libhymba_hh.so")

HH_F32, HH_BF16 = 0, 1
HH_WS = ["Q", "K", "V", "XS", "Z", "DELTA", "BC", "O", "Y", "F", "SCAN", "GEMM", "SSQ"]
STATUS = {0: "HH_OK", 1: "HH_ERR_INVALID_ARG", 2: "HH_ERR_UNSUPPORTED",
          3: "HH_ERR_WORKSPACE", 4: "HH_ERR_HIP"}
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


class HHDims(ctypes.Structure):
    _fields_ = [("d_model", _i32), ("n_heads", _i32), ("n_kv_heads", _i32), ("head_dim", _i32),
                ("d_inner", _i32), ("d_state", _i32), ("d_conv", _i32), ("n_meta", _i32),
                ("dtype", _i32), ("rms_eps", ctypes.c_float), ("rope_base", ctypes.c_float),
                ("ssm_heads", _i32)]


class HHWeights(ctypes.Structure):
    _fields_ = [("w_in", _vp), ("dt_bias", _vp), ("A", _vp), ("conv_w", _vp), ("conv_b", _vp),
                ("beta_attn", _vp), ("beta_ssm", _vp), ("w_out", _vp), ("kv_producer", _i32)]


class HHMeta(ctypes.Structure):
    _fields_ = [("k", _vp), ("v", _vp), ("h0", _vp), ("conv_tail", _vp)]


class HHKV(ctypes.Structure):
    _fields_ = [("full_k", _vp), ("full_v", _vp), ("cache_k", _vp), ("cache_v", _vp),
                ("len", _vp), ("cap", _i32), ("is_ring", _i32)]


class HHSsmState(ctypes.Structure):
    _fields_ = [("h", _vp), ("conv", _vp)]


class HHBlockWeights(ctypes.Structure):
    _fields_ = [("mixer", HHWeights), ("norm1", _vp), ("norm2", _vp), ("w_gate_up", _vp),
                ("w_down", _vp), ("d_ff", _i32)]


class HHStageTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", _i32), ("total_ms", ctypes.c_double)]


class HHError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libhymba_hh.so (built in-tree); raise if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -m hybrid_attention_ssm_amd.csrc.build)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.hh_version.restype = ctypes.c_char_p
        L.hh_last_error.restype = ctypes.c_char_p
        L.hh_meta_prefix_workspace_size.restype = ctypes.c_size_t
        L.hh_meta_prefix_workspace_size.argtypes = [P(HHDims), _i32]
        L.hh_prefill_workspace_size.restype = ctypes.c_size_t
        L.hh_prefill_workspace_size.argtypes = [P(HHDims), _i32, _i32, _i32]
        L.hh_prefill_workspace_layout.restype = ctypes.c_size_t
        L.hh_prefill_workspace_layout.argtypes = [P(HHDims), _i32, _i32, _i32, P(ctypes.c_size_t)]
        L.hh_decode_workspace_size.restype = ctypes.c_size_t
        L.hh_decode_workspace_size.argtypes = [P(HHDims), _i32, _i32, _i32]
        L.hh_meta_prefix.restype = ctypes.c_int
        L.hh_meta_prefix.argtypes = [P(HHDims), P(HHWeights), _vp, _vp, _vp, _vp, _vp, _vp,
                                     ctypes.c_size_t, _vp]
        L.hh_prefill.restype = ctypes.c_int
        L.hh_prefill.argtypes = [P(HHDims), P(HHWeights), _vp, _i32, _i32, P(HHMeta), _i32, _i32,
                                 _vp, P(HHKV), P(HHSsmState), _vp, ctypes.c_size_t, _vp]
        L.hh_decode_step.restype = ctypes.c_int
        L.hh_decode_step.argtypes = [P(HHDims), P(HHWeights), _vp, _i32, P(HHMeta), _i32, _i32,
                                     P(HHKV), P(HHSsmState), _vp, _vp, ctypes.c_size_t, _vp]
        L.hh_decode_step_noalloc.restype = ctypes.c_int
        L.hh_decode_step_noalloc.argtypes = [P(HHDims), P(HHWeights), _vp, _i32, P(HHMeta), _i32, _i32,
                                             P(HHKV), P(HHSsmState), _vp, _vp]
        L.hh_block_meta_prefix_workspace_size.restype = ctypes.c_size_t
        L.hh_block_meta_prefix_workspace_size.argtypes = [P(HHDims), _i32]
        L.hh_block_prefill_workspace_size.restype = ctypes.c_size_t
        L.hh_block_prefill_workspace_size.argtypes = [P(HHDims), _i32, _i32, _i32, _i32]
        L.hh_block_decode_workspace_size.restype = ctypes.c_size_t
        L.hh_block_decode_workspace_size.argtypes = [P(HHDims), _i32, _i32, _i32, _i32]
        L.hh_block_meta_prefix.restype = ctypes.c_int
        L.hh_block_meta_prefix.argtypes = [P(HHDims), P(HHBlockWeights), _vp, _vp, _vp, _vp, _vp,
                                           _vp, ctypes.c_size_t, _vp]
        L.hh_block_prefill.restype = ctypes.c_int
        L.hh_block_prefill.argtypes = [P(HHDims), P(HHBlockWeights), _vp, _i32, _i32, P(HHMeta),
                                       _i32, _i32, _vp, P(HHKV), P(HHSsmState), _vp,
                                       ctypes.c_size_t, _vp]
        L.hh_block_decode_step.restype = ctypes.c_int
        L.hh_block_decode_step.argtypes = [P(HHDims), P(HHBlockWeights), _vp, _i32, P(HHMeta),
                                           _i32, _i32, P(HHKV), P(HHSsmState), _vp, _vp,
                                           ctypes.c_size_t, _vp]
        L.hh_stage_attn.restype = ctypes.c_int
        L.hh_stage_attn.argtypes = [P(HHDims), _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp]
        L.hh_stage_ssm_workspace_size.restype = ctypes.c_size_t
        L.hh_stage_ssm_workspace_size.argtypes = [P(HHDims), _i32, _i32]
        L.hh_stage_ssm.restype = ctypes.c_int
        L.hh_stage_ssm.argtypes = [P(HHDims), P(HHWeights), _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                   _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.hh_timing_enable.restype = ctypes.c_int
        L.hh_timing_enable.argtypes = [_i32]
        L.hh_timing_read.restype = _i32
        L.hh_timing_read.argtypes = [ctypes.POINTER(HHStageTime), _i32]
        _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        raise HHError(fn, status, lib().hh_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libhymba_hh must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def storage_dtype(dims: LayerDims) -> torch.dtype:
    return torch.bfloat16 if dims.dtype == "bf16" else torch.float32


def hh_dims(dims: LayerDims) -> HHDims:
    return HHDims(dims.d_model, dims.n_heads, dims.n_kv_heads, dims.head_dim, dims.d_inner,
                  dims.d_state, dims.d_conv, dims.n_meta,
                  HH_BF16 if dims.dtype == "bf16" else HH_F32, dims.eps, dims.rope_base,
                  dims.ssm_heads)


def hh_version() -> str:
    return lib().hh_version().decode()


def hh_last_error() -> str:
    return lib().hh_last_error().decode()


# --------------------------------------------------------------------------
# device-side parameter bundles
# --------------------------------------------------------------------------
@dataclass
class DeviceLayer:
    dims: LayerDims
    tensors: dict
    struct: HHWeights

    @property
    def kv_producer(self) -> bool:
        return bool(self.struct.kv_producer)


def upload_weights(dims: LayerDims, w: dict, device="cuda") -> DeviceLayer:
    """Copy one layer's parameters (numpy, from synth.layer_weights) to the GPU."""
    sd = storage_dtype(dims)
    f32 = torch.float32
    t = {
        "w_in": torch.as_tensor(w["w_in"]).to(device=device, dtype=sd).contiguous(),
        "dt_bias": torch.as_tensor(w["dt_bias"]).to(device=device, dtype=f32).contiguous(),
        "A": torch.as_tensor(w["A"]).to(device=device, dtype=f32).contiguous(),
        "conv_w": torch.as_tensor(w["conv_w"]).to(device=device, dtype=f32).contiguous(),
        "conv_b": torch.as_tensor(w["conv_b"]).to(device=device, dtype=f32).contiguous(),
        "beta_attn": torch.as_tensor(w["beta_attn"]).to(device=device, dtype=f32).contiguous(),
        "beta_ssm": torch.as_tensor(w["beta_ssm"]).to(device=device, dtype=f32).contiguous(),
        "w_out": torch.as_tensor(w["w_out"]).to(device=device, dtype=sd).contiguous(),
    }
    st = HHWeights(_ptr(t["w_in"]), _ptr(t["dt_bias"]), _ptr(t["A"]), _ptr(t["conv_w"]),
                   _ptr(t["conv_b"]), _ptr(t["beta_attn"]), _ptr(t["beta_ssm"]),
                   _ptr(t["w_out"]), 1 if w.get("kv_producer", True) else 0)
    return DeviceLayer(dims, t, st)


@dataclass
class DeviceBlock:
    dims: LayerDims
    mixer: DeviceLayer
    tensors: dict
    struct: HHBlockWeights

    @property
    def kv_producer(self) -> bool:
        return self.mixer.kv_producer

    @property
    def d_ff(self) -> int:
        return int(self.struct.d_ff)


def upload_block_weights(dims: LayerDims, bw: dict, device="cuda") -> DeviceBlock:
    """Copy one block's parameters (numpy, from synth.block_weights) to the GPU."""
    sd = storage_dtype(dims)
    mixer = upload_weights(dims, bw["mixer"], device)
    t = {"norm1": torch.as_tensor(bw["norm1"]).to(device=device, dtype=torch.float32).contiguous(),
         "norm2": torch.as_tensor(bw["norm2"]).to(device=device, dtype=torch.float32).contiguous(),
         "w_gate_up": torch.as_tensor(bw["w_gate_up"]).to(device=device, dtype=sd).contiguous(),
         "w_down": torch.as_tensor(bw["w_down"]).to(device=device, dtype=sd).contiguous()}
    st = HHBlockWeights(mixer.struct, _ptr(t["norm1"]), _ptr(t["norm2"]), _ptr(t["w_gate_up"]),
                        _ptr(t["w_down"]), int(bw["d_ff"]))
    return DeviceBlock(dims, mixer, t, st)


class Workspace:
    """A growable device scratch buffer (one per device and user)."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes: int, device) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != torch.device(device):
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        return self.buf


_default_ws = Workspace()


# --------------------------------------------------------------------------
# entry points
# --------------------------------------------------------------------------
def hh_meta_prefix_workspace_size(dims: LayerDims, kv_producer=True) -> int:
    d = hh_dims(dims)
    return lib().hh_meta_prefix_workspace_size(ctypes.byref(d), int(bool(kv_producer)))


def hh_prefill_workspace_size(dims: LayerDims, batch: int, seqlen: int, kv_producer=True) -> int:
    d = hh_dims(dims)
    return lib().hh_prefill_workspace_size(ctypes.byref(d), batch, seqlen, int(bool(kv_producer)))


def hh_prefill_workspace_layout(dims: LayerDims, batch: int, seqlen: int, kv_producer=True) -> dict:
    d = hh_dims(dims)
    offs = (ctypes.c_size_t * len(HH_WS))()
    total = lib().hh_prefill_workspace_layout(ctypes.byref(d), batch, seqlen,
                                              int(bool(kv_producer)), offs)
    out = {name: (None if offs[i] == ctypes.c_size_t(-1).value else int(offs[i]))
           for i, name in enumerate(HH_WS)}
    out["total"] = int(total)
    return out


def hh_decode_workspace_size(dims: LayerDims, batch: int, cap: int, kv_producer=True) -> int:
    d = hh_dims(dims)
    return lib().hh_decode_workspace_size(ctypes.byref(d), batch, cap, int(bool(kv_producer)))


def hh_meta_prefix(layer: DeviceLayer, meta_tokens: torch.Tensor, out: Optional[dict] = None,
                   ws: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Meta K/V [G, m, hd], h0 [D, N] fp32 and conv tail [k-1, D] of one layer."""
    dims = layer.dims
    dev = meta_tokens.device
    sd = storage_dtype(dims)
    G, m, hd, D, N, k = (dims.n_kv_heads, dims.n_meta, dims.head_dim, dims.d_inner,
                         dims.d_state, dims.d_conv)
    if out is None:
        out = {"h0": torch.empty(D, N, dtype=torch.float32, device=dev),
               "conv_tail": torch.empty(k - 1, D, dtype=torch.float32, device=dev)}
        if layer.kv_producer:
            out["k"] = torch.empty(G, m, hd, dtype=sd, device=dev)
            out["v"] = torch.empty(G, m, hd, dtype=sd, device=dev)
    need = hh_meta_prefix_workspace_size(dims, layer.kv_producer)
    if ws is None:
        ws = _default_ws.get(need, dev)
    d = hh_dims(dims)
    _check("hh_meta_prefix", lib().hh_meta_prefix(
        ctypes.byref(d), ctypes.byref(layer.struct), _ptr(meta_tokens), _ptr(out.get("k")),
        _ptr(out.get("v")), _ptr(out["h0"]), _ptr(out["conv_tail"]), _ptr(ws), ws.numel(),
        _stream(stream)))
    return out


def make_meta(k, v, h0, conv_tail) -> HHMeta:
    return HHMeta(_ptr(k), _ptr(v), _ptr(h0), _ptr(conv_tail))


def make_kv(full_k=None, full_v=None, cache_k=None, cache_v=None, length=None, cap=0,
            is_ring=False) -> HHKV:
    return HHKV(_ptr(full_k), _ptr(full_v), _ptr(cache_k), _ptr(cache_v), _ptr(length),
                int(cap), int(bool(is_ring)))


def hh_prefill(layer: DeviceLayer, x: torch.Tensor, meta: HHMeta, window: int, is_global: bool,
               out: torch.Tensor, kv: Optional[HHKV] = None, state_h: Optional[torch.Tensor] = None,
               state_conv: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
               stream=None) -> None:
    """hh_prefill on device tensors; x [B, n, d] -> out [B, n, d]."""
    B, n, _ = x.shape
    need = hh_prefill_workspace_size(layer.dims, B, n, layer.kv_producer)
    if ws is None:
        ws = _default_ws.get(need, x.device)
    d = hh_dims(layer.dims)
    st = HHSsmState(_ptr(state_h), _ptr(state_conv))
    _check("hh_prefill", lib().hh_prefill(
        ctypes.byref(d), ctypes.byref(layer.struct), _ptr(x), B, n, ctypes.byref(meta),
        int(window), int(bool(is_global)), _ptr(out), ctypes.byref(kv) if kv is not None else None,
        ctypes.byref(st), _ptr(ws), ws.numel(), _stream(stream)))


def hh_stage_attn(dims: LayerDims, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  meta_k: Optional[torch.Tensor], meta_v: Optional[torch.Tensor], window: int,
                  is_global: bool, o: torch.Tensor, stream=None) -> None:
    """hh_stage_attn: q [B, n, H*hd], k/v [B, G, n, hd], meta k/v [G, m, hd] -> o [B, n, H*hd]."""
    B, n = q.shape[0], q.shape[1]
    d = hh_dims(dims)
    _check("hh_stage_attn", lib().hh_stage_attn(
        ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(meta_k), _ptr(meta_v), B, n, int(window),
        int(bool(is_global)), _ptr(o), _stream(stream)))


def hh_stage_ssm_workspace_size(dims: LayerDims, batch: int, seqlen: int) -> int:
    d = hh_dims(dims)
    return lib().hh_stage_ssm_workspace_size(ctypes.byref(d), batch, seqlen)


def hh_stage_ssm(layer: DeviceLayer, xs: torch.Tensor, z: torch.Tensor, delta: torch.Tensor,
                 bc: torch.Tensor, h0: Optional[torch.Tensor], conv_tail: Optional[torch.Tensor],
                 batch: int, seqlen: int, y: Optional[torch.Tensor], h_out: Optional[torch.Tensor],
                 tail_out: Optional[torch.Tensor], ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """hh_stage_ssm: xs/z/delta in the channel-block-major layout, bc [B*n, 2N] ->
    y [B*n, D], h_out [B, D, N], tail_out [B, k-1, D]."""
    need = hh_stage_ssm_workspace_size(layer.dims, batch, seqlen)
    if ws is None:
        ws = _default_ws.get(need, xs.device)
    d = hh_dims(layer.dims)
    _check("hh_stage_ssm", lib().hh_stage_ssm(
        ctypes.byref(d), ctypes.byref(layer.struct), _ptr(xs), _ptr(z), _ptr(delta), _ptr(bc), _ptr(h0),
        _ptr(conv_tail), batch, seqlen, _ptr(y), _ptr(h_out), _ptr(tail_out), _ptr(ws), ws.numel(),
        _stream(stream)))


def hh_decode_step(layer: DeviceLayer, x_t: torch.Tensor, meta: HHMeta, window: int,
                   is_global: bool, kv: HHKV, state_h: torch.Tensor, state_conv: torch.Tensor,
                   out: torch.Tensor, ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """hh_decode_step on device tensors; x_t [B, d] -> out [B, d]."""
    B = x_t.shape[0]
    need = hh_decode_workspace_size(layer.dims, B, kv.cap, layer.kv_producer)
    if ws is None:
        ws = _default_ws.get(need, x_t.device)
    d = hh_dims(layer.dims)
    st = HHSsmState(_ptr(state_h), _ptr(state_conv))
    _check("hh_decode_step", lib().hh_decode_step(
        ctypes.byref(d), ctypes.byref(layer.struct), _ptr(x_t), B, ctypes.byref(meta),
        int(window), int(bool(is_global)), ctypes.byref(kv), ctypes.byref(st), _ptr(out),
        _ptr(ws), ws.numel(), _stream(stream)))


def hh_decode_step_noalloc(layer: DeviceLayer, x_t: torch.Tensor, meta: HHMeta, window: int,
                           is_global: bool, kv: HHKV, state_h: torch.Tensor, state_conv: torch.Tensor,
                           out: torch.Tensor, stream=None) -> None:
    """hh_decode_step_noalloc on device tensors (the library's static scratch,
    no workspace); x_t [B, d] -> out [B, d]."""
    B = x_t.shape[0]
    d = hh_dims(layer.dims)
    st = HHSsmState(_ptr(state_h), _ptr(state_conv))
    _check("hh_decode_step_noalloc", lib().hh_decode_step_noalloc(
        ctypes.byref(d), ctypes.byref(layer.struct), _ptr(x_t), B, ctypes.byref(meta),
        int(window), int(bool(is_global)), ctypes.byref(kv), ctypes.byref(st), _ptr(out),
        _stream(stream)))


def to_device(a: np.ndarray, dtype: torch.dtype, device="cuda") -> torch.Tensor:
    return torch.as_tensor(np.ascontiguousarray(a)).to(device=device, dtype=dtype).contiguous()


def hh_timing_enable(on: bool = True) -> None:
    _check("hh_timing_enable", lib().hh_timing_enable(int(bool(on))))


def hh_timing_read(max_stages: int = 32) -> dict:
    """{stage: (launches, total_ms)} since the last read; clears the record."""
    buf = (HHStageTime * max_stages)()
    n = lib().hh_timing_read(buf, max_stages)
    if n < 0:
        raise HHError("hh_timing_read", 4, "HIP error while reading stage events")
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(n)}


# --------------------------------------------------------------------------
# the block around the layer
# --------------------------------------------------------------------------
def hh_block_meta_prefix(block: DeviceBlock, meta_tokens: torch.Tensor, ws=None, stream=None) -> dict:
    """hh_block_meta_prefix: the layer's meta part for the block input R."""
    dims = block.dims
    dev = meta_tokens.device
    sd = storage_dtype(dims)
    G, m, hd, D, N, k = (dims.n_kv_heads, dims.n_meta, dims.head_dim, dims.d_inner,
                         dims.d_state, dims.d_conv)
    out = {"h0": torch.empty(D, N, dtype=torch.float32, device=dev),
           "conv_tail": torch.empty(k - 1, D, dtype=torch.float32, device=dev)}
    if block.kv_producer:
        out["k"] = torch.empty(G, m, hd, dtype=sd, device=dev)
        out["v"] = torch.empty(G, m, hd, dtype=sd, device=dev)
    d = hh_dims(dims)
    need = lib().hh_block_meta_prefix_workspace_size(ctypes.byref(d), int(block.kv_producer))
    if ws is None:
        ws = _default_ws.get(need, dev)
    _check("hh_block_meta_prefix", lib().hh_block_meta_prefix(
        ctypes.byref(d), ctypes.byref(block.struct), _ptr(meta_tokens), _ptr(out.get("k")),
        _ptr(out.get("v")), _ptr(out["h0"]), _ptr(out["conv_tail"]), _ptr(ws), ws.numel(),
        _stream(stream)))
    return out


def hh_block_prefill_workspace_size(block: DeviceBlock, batch: int, seqlen: int) -> int:
    d = hh_dims(block.dims)
    return lib().hh_block_prefill_workspace_size(ctypes.byref(d), block.d_ff, batch, seqlen,
                                                 int(block.kv_producer))


def hh_block_decode_workspace_size(block: DeviceBlock, batch: int, cap: int) -> int:
    d = hh_dims(block.dims)
    return lib().hh_block_decode_workspace_size(ctypes.byref(d), block.d_ff, batch, cap,
                                                int(block.kv_producer))


def hh_block_prefill(block: DeviceBlock, x: torch.Tensor, meta: HHMeta, window: int,
                     is_global: bool, out: torch.Tensor, kv: Optional[HHKV] = None,
                     state_h: Optional[torch.Tensor] = None,
                     state_conv: Optional[torch.Tensor] = None, ws=None, stream=None) -> None:
    """hh_block_prefill on device tensors; x [B, n, d] -> out [B, n, d]."""
    B, n, _ = x.shape
    if ws is None:
        ws = _default_ws.get(hh_block_prefill_workspace_size(block, B, n), x.device)
    d = hh_dims(block.dims)
    st = HHSsmState(_ptr(state_h), _ptr(state_conv))
    _check("hh_block_prefill", lib().hh_block_prefill(
        ctypes.byref(d), ctypes.byref(block.struct), _ptr(x), B, n, ctypes.byref(meta),
        int(window), int(bool(is_global)), _ptr(out), ctypes.byref(kv) if kv is not None else None,
        ctypes.byref(st), _ptr(ws), ws.numel(), _stream(stream)))


def hh_block_decode_step(block: DeviceBlock, x_t: torch.Tensor, meta: HHMeta, window: int,
                         is_global: bool, kv: HHKV, state_h: torch.Tensor,
                         state_conv: torch.Tensor, out: torch.Tensor, ws=None, stream=None) -> None:
    """hh_block_decode_step on device tensors; x_t [B, d] -> out [B, d]."""
    B = x_t.shape[0]
    if ws is None:
        ws = _default_ws.get(hh_block_decode_workspace_size(block, B, kv.cap), x_t.device)
    d = hh_dims(block.dims)
    st = HHSsmState(_ptr(state_h), _ptr(state_conv))
    _check("hh_block_decode_step", lib().hh_block_decode_step(
        ctypes.byref(d), ctypes.byref(block.struct), _ptr(x_t), B, ctypes.byref(meta),
        int(window), int(bool(is_global)), ctypes.byref(kv), ctypes.byref(st), _ptr(out),
        _ptr(ws), ws.numel(), _stream(stream)))

