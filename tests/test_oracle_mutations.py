"""Plant plausible mistakes in the oracle (CPU only) and check that the pins
catch each one: the library-composition pin must disagree for every mutant."""
import numpy as np
import pytest

from oracle import hymba_ref as ref
from tests.test_oracle_pins import GQA, _layer, layer_by_library


def _max_err(window=7, is_global=False):
    dims = GQA
    x, R, w = _layer(dims, 30, seed=21)
    got = ref.prefill(dims.as_dict(), w, R, x, window, is_global)
    want = layer_by_library(dims, w, R, x[0], window, is_global)
    return float(np.abs(got["out"][0] - want["out"]).max())


_orig_split = ref.split_projection
_orig_attend = ref.attend
_orig_scan = ref.selective_scan
_orig_conv = ref.causal_conv


def _swap_xs_z(P, dims, kv_producer=True):
    p = _orig_split(P, dims, kv_producer)
    p["xs"], p["z"] = p["z"], p["xs"]
    return p


def _swap_b_c(P, dims, kv_producer=True):
    p = _orig_split(P, dims, kv_producer)
    p["B"], p["C"] = p["C"], p["B"]
    return p


def _no_scale(q, K, V, rows, scale):
    return _orig_attend(q, K, V, rows, 1.0)


def _kv_swapped(q, K, V, rows, scale):
    return _orig_attend(q, V, K, rows, scale)


def _group_interleaved(q, K, V, rows, scale):
    H, G = q.shape[0], K.shape[1]
    perm = np.arange(H) % G                   # wrong head -> group map
    out = np.empty_like(q)
    for h in range(H):
        o, _ = _orig_attend(q[h:h + 1], K[:, perm[h]:perm[h] + 1], V[:, perm[h]:perm[h] + 1], rows, scale)
        out[h] = o[0]
    return out, None


def _window_off_by_one(i, m, window, is_global):
    lo = m if is_global else max(m, i - window)
    return np.concatenate([np.arange(m), np.arange(lo, i + 1)]).astype(np.int64)


def _no_meta_keys(i, m, window, is_global):
    lo = m if is_global else max(m, i - window + 1)
    return np.arange(lo, i + 1).astype(np.int64)


def _scan_no_delta_in_input(u, delta, A, Bm, Cm, h):
    return _orig_scan(u / np.where(delta == 0, 1, delta), delta, A, Bm, Cm, h)


def _scan_positive_exponent(u, delta, A, Bm, Cm, h):
    return _orig_scan(u, delta, -A * 0.5, Bm, Cm, h)


def _conv_taps_not_reversed(xs, conv_w, conv_b, history):
    return _orig_conv(xs, conv_w[:, ::-1], conv_b, history)


MUTANTS = {
    "xs<->z": ("split_projection", _swap_xs_z),
    "B<->C": ("split_projection", _swap_b_c),
    "no 1/sqrt(hd)": ("attend", _no_scale),
    "K<->V": ("attend", _kv_swapped),
    "head->group map": ("attend", _group_interleaved),
    "window off by one": ("allowed_rows", _window_off_by_one),
    "meta keys dropped": ("allowed_rows", _no_meta_keys),
    "Delta missing from input term": ("selective_scan", _scan_no_delta_in_input),
    "wrong decay": ("selective_scan", _scan_positive_exponent),
    "conv taps not reversed": ("causal_conv", _conv_taps_not_reversed),
    "softplus -> exp": ("softplus", np.exp),
    "silu -> sigmoid": ("silu", lambda v: 0.5 * (1.0 + np.tanh(0.5 * v))),
    "no eps / sum not mean": ("rms_normalize", lambda v, eps: v / np.sqrt(np.sum(v * v, axis=-1, keepdims=True))),
    "sum not average": ("fuse", lambda O, Y, b1, b2, eps: 2.0 * ref.__dict__["_fuse_orig"](O, Y, b1, b2, eps)),
}
ref._fuse_orig = ref.fuse


# the block around the layer: caught by the block's library-composition pin
from tests.test_oracle_pins import _block, block_by_library


def _block_err():
    from hybrid_attention_ssm_amd.configs import TINY
    x, R, bw = _block(TINY, 13, seed=34)
    got = ref.block_prefill(TINY.as_dict(), bw, R, x, 6, False)
    want = block_by_library(TINY, bw, R, x[0], 6, False)
    return float(np.abs(got["out"][0] - want["out"]).max())


_orig_mlp = ref.mlp
_orig_rms_norm = ref.rms_norm
BLOCK_MUTANTS = {
    "gate<->up": ("mlp", lambda v, w_gu, w_down, store=None:
                  _orig_mlp(v, w_gu[np.arange(w_gu.shape[0]) ^ 1], w_down)),
    "MLP without SiLU": ("mlp", lambda v, w_gu, w_down, store=None:
                         ((np.asarray(v) @ w_gu.T)[..., 0::2] * (np.asarray(v) @ w_gu.T)[..., 1::2]) @ w_down.T),
    "norm gain dropped": ("rms_norm", lambda v, g, eps: _orig_rms_norm(v, np.ones_like(g), eps)),
    "norm gain applied twice": ("rms_norm", lambda v, g, eps: np.asarray(g) * _orig_rms_norm(v, g, eps)),
}


def _block_store_err():
    from tests.test_oracle_pins import _block, block_by_library
    from hybrid_attention_ssm_amd.configs import TINY
    from hybrid_attention_ssm_amd.synth import round_bf16
    x, R, bw = _block(TINY, 13, seed=37)
    got = ref.block_prefill(TINY.as_dict(), bw, R, x, 6, False, store=round_bf16)
    want = block_by_library(TINY, bw, R, x[0], 6, False, store=round_bf16)
    return float(np.abs(got["out"][0] - want["out"]).max())


STORE_MUTANTS = {
    # the MLP's hidden units handed on unrounded
    "MLP hidden not stored": ("mlp", lambda v, w_gu, w_down, store=None: _orig_mlp(v, w_gu, w_down)),
    # the rounding applied to the hidden units twice over a wider type: the
    # gate rounded before the product instead of the product
    "MLP gate stored instead of the product": (
        "mlp", lambda v, w_gu, w_down, store=None: (
            np.asarray(store(ref.silu((np.asarray(v) @ w_gu.T)[..., 0::2])), dtype=np.float64)
            * (np.asarray(v) @ w_gu.T)[..., 1::2]) @ w_down.T),
}


def test_unmutated_block_store_agrees():
    assert _block_store_err() < 1e-9


@pytest.mark.parametrize("name", sorted(STORE_MUTANTS))
def test_block_store_pin_catches_mutant(name, monkeypatch):
    attr, fn = STORE_MUTANTS[name]
    monkeypatch.setattr(ref, attr, fn)
    assert _block_store_err() > 1e-4, f"mutant '{name}' not caught"


def test_unmutated_block_agrees():
    assert _block_err() < 1e-9


@pytest.mark.parametrize("name", sorted(BLOCK_MUTANTS))
def test_block_pin_catches_mutant(name, monkeypatch):
    attr, fn = BLOCK_MUTANTS[name]
    monkeypatch.setattr(ref, attr, fn)
    assert _block_err() > 1e-4, f"mutant '{name}' not caught"


def test_unmutated_oracle_agrees():
    assert _max_err() < 1e-9


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ref, attr, fn)
    assert _max_err() > 1e-4, f"mutant '{name}' not caught"


# rotary embedding: caught by the library composition (complex multiplication)
from dataclasses import replace as _replace

_orig_rope = ref.rope


def _rope_err():
    from tests.test_oracle_pins import GQA_ROPE
    x, R, w = _layer(GQA_ROPE, 26, seed=43)
    got = ref.prefill(GQA_ROPE.as_dict(), w, R, x, 7, False)
    want = layer_by_library(GQA_ROPE, w, R, x[0], 7, False)
    return float(np.abs(got["out"][0] - want["out"]).max())


def _rope_adjacent_pairs(v, pos, base):
    v = np.asarray(v, dtype=np.float64)
    hd = v.shape[-1]
    perm = np.concatenate([np.arange(0, hd, 2), np.arange(1, hd, 2)])   # (2i, 2i+1) pairs
    inv = np.argsort(perm)
    return _orig_rope(v[..., perm], pos, base)[..., inv]


def _rope_half_frequency_exponent(v, pos, base):
    return _orig_rope(v, pos, base ** 0.5)


ROPE_MUTANTS = {
    "rope turns the other way": lambda v, pos, base: _orig_rope(v, -np.asarray(pos), base),
    "rope pairs adjacent dims": _rope_adjacent_pairs,
    "rope frequency exponent halved": _rope_half_frequency_exponent,
    "rope positions without the meta rows": lambda v, pos, base: _orig_rope(
        v, np.maximum(np.asarray(pos) - 3, 0), base),
}


def test_unmutated_rope_agrees():
    assert _rope_err() < 1e-9


@pytest.mark.parametrize("name", sorted(ROPE_MUTANTS))
def test_rope_pin_catches_mutant(name, monkeypatch):
    monkeypatch.setattr(ref, "rope", ROPE_MUTANTS[name])
    assert _rope_err() > 1e-4, f"mutant '{name}' not caught"


# Mamba2 heads: caught by the library composition (SSD matrix form)
_orig_ssm_params = ref.ssm_params


def _m2_err():
    from tests.test_oracle_pins import GQA_M2
    x, R, w = _layer(GQA_M2, 26, seed=46)
    got = ref.prefill(GQA_M2.as_dict(), w, R, x, 7, False)
    want = layer_by_library(GQA_M2, w, R, x[0], 7, False)
    return float(np.abs(got["out"][0] - want["out"]).max())


def _m2_interleaved_heads(delta, A, dims):
    S = dict(dims).get("ssm_heads", 0)
    if not S:
        return _orig_ssm_params(delta, A, dims)
    D, N = dict(dims)["d_inner"], dict(dims)["d_state"]
    head = np.arange(D) % S                      # channel c -> head c % S instead of c // P
    return np.asarray(delta, dtype=np.float64)[..., head], np.repeat(np.asarray(A, np.float64)[head][:, None], N, axis=1)


def _m2_first_head_decay(delta, A, dims):
    d, a = _orig_ssm_params(delta, A, dims)
    return d, np.full_like(a, a[0, 0])           # every head decays like head 0


M2_MUTANTS = {"Mamba2 heads interleaved": _m2_interleaved_heads,
              "Mamba2 decay of head 0 everywhere": _m2_first_head_decay}


def test_unmutated_mamba2_agrees():
    assert _m2_err() < 1e-9


@pytest.mark.parametrize("name", sorted(M2_MUTANTS))
def test_mamba2_pin_catches_mutant(name, monkeypatch):
    monkeypatch.setattr(ref, "ssm_params", M2_MUTANTS[name])
    assert _m2_err() > 1e-4, f"mutant '{name}' not caught"
