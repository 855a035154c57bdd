"""Pins for the CPU oracle, independent of the oracle's own code.

Each test checks the oracle against something it does not share code with:
hand-derived values (tests/golden), closed forms, invariants the Hymba paper's
equations imply, or the layer composed from library routines (torch CPU in
fp64: linear, conv1d, scaled_dot_product_attention with an explicit boolean
mask, softplus, silu, rms_norm) with the SSM written in the alternative
alpha-matrix form of Eq. (2).  CPU only.
"""
import math
import os

import numpy as np
from dataclasses import replace
import pytest
import torch
import torch.nn.functional as TF

from oracle import hymba_ref as ref
from hybrid_attention_ssm_amd.configs import TINY, LayerDims
from hybrid_attention_ssm_amd.synth import layer_weights

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(v) for v in line.split()])
    return rows


def _layer(dims: LayerDims, n, seed, kv_producer=True, batch=1):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((batch, n, dims.d_model)).astype(np.float32)
    R = rng.standard_normal((dims.n_meta, dims.d_model)).astype(np.float32)
    w = layer_weights(rng, dims, kv_producer)
    return x, R, w


GQA = LayerDims(d_model=48, n_heads=4, n_kv_heads=2, head_dim=8, d_inner=24,
                d_state=4, d_conv=4, n_meta=3, dtype="f32")


# ---------------------------------------------------------------------------
# the layer composed from library routines; SSM via Eq. (2)'s alpha matrix
# ---------------------------------------------------------------------------
def rope_by_complex(v, pos, base):
    """RoPE as complex multiplication: (v_i + j v_{i+hd/2}) * e^{j pos f_i} with
    f_i = base^(-2i/hd), real and imaginary parts back in the two halves."""
    v = torch.as_tensor(np.asarray(v, dtype=np.float64)) if not torch.is_tensor(v) else v
    half = v.shape[-1] // 2
    f = torch.tensor(float(base), dtype=torch.float64) ** (
        -2.0 * torch.arange(half, dtype=torch.float64) / v.shape[-1])
    ang = torch.as_tensor(pos, dtype=torch.float64)[..., None] * f
    z = torch.complex(v[..., :half], v[..., half:]) * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([z.real, z.imag], dim=-1)


def layer_by_library(dims: LayerDims, w, R, xb, window, is_global):
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    m, n = R.shape[0], xb.shape[0]
    T = m + n
    H, G, hd, D, N, k = (dims.n_heads, dims.n_kv_heads, dims.head_dim,
                         dims.d_inner, dims.d_state, dims.d_conv)
    Xt = torch.cat([t(R), t(xb)])
    P = TF.linear(Xt, t(w["w_in"]))
    S = dims.ssm_heads
    q, kk, v, xs, z, dt, Bm, Cm = torch.split(
        P, [H * hd, G * hd, G * hd, D, D, S or D, N, N], dim=-1)
    if dims.rope_base:
        q = rope_by_complex(q.view(T, H, hd), torch.arange(T)[:, None], dims.rope_base).reshape(T, H * hd)
        kk = rope_by_complex(kk.view(T, G, hd), torch.arange(T)[:, None], dims.rope_base).reshape(T, G * hd)
    # A-shape mask: meta keys always, real keys in the window (or causal)
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    real = (j >= m) & (j <= i) & ((i - j < window) | is_global)
    mask = (j < m) | real
    qh = q.view(T, H, hd).transpose(0, 1)
    kh = kk.view(T, G, hd).transpose(0, 1).repeat_interleave(H // G, dim=0)
    vh = v.view(T, G, hd).transpose(0, 1).repeat_interleave(H // G, dim=0)
    O = TF.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask)
    O = O.transpose(0, 1).reshape(T, H * hd)
    c = TF.conv1d(xs.T[None], t(w["conv_w"])[:, None, :], t(w["conv_b"]),
                  padding=k - 1, groups=D)[0, :, :T].T
    u = TF.silu(c)
    delta = TF.softplus(dt + t(w["dt_bias"]), threshold=1e4)
    A = t(w["A"])
    cs = torch.cumsum(delta, 0)                       # sum_{k<=i} Delta_k
    y = torch.zeros(T, D, dtype=torch.float64)
    hT = torch.zeros(D, N, dtype=torch.float64)
    lower = (j <= i)
    if S:
        # Mamba2 heads in the SSD matrix form: per head a scalar decay, so
        # y = ((C B^T) o L o Delta_tau) u with L[i, j] = exp(A_h sum_{k=j+1..i} Delta_k)
        Pc = D // S
        CB = Cm @ Bm.T                                    # [T, T]
        for hh in range(S):
            diff = torch.where(lower, cs[:, hh][:, None] - cs[:, hh][None, :], torch.zeros(()))
            Lm = torch.where(lower, torch.exp(A[hh] * diff), torch.zeros(()))
            M = CB * Lm * delta[:, hh][None, :]
            cols = slice(hh * Pc, (hh + 1) * Pc)
            y[:, cols] = M @ u[:, cols]
            wT = torch.exp(A[hh] * (cs[-1, hh] - cs[:, hh])) * delta[:, hh]     # [T]
            hT[cols] = (u[:, cols] * wT[:, None]).T @ Bm
        D_loop = 0
    else:
        D_loop = D
    for ch in range(D_loop):
        # prod_{k=j+1..i} exp(A Delta_k) = exp(A (cs_i - cs_j)) for j <= i
        diff = torch.where(lower, cs[:, ch][:, None] - cs[:, ch][None, :], torch.zeros(()))
        E = torch.exp(A[ch][None, None, :] * diff[:, :, None])          # [T, T, N]
        alpha = torch.einsum("is,ijs,js->ij", Cm, E, Bm) * delta[:, ch][None, :]
        alpha = torch.where(lower, alpha, torch.zeros(()))
        y[:, ch] = alpha @ u[:, ch]
        ET = torch.exp(A[ch][None, :] * (cs[-1, ch] - cs[:, ch])[:, None])  # [T, N]
        hT[ch] = (ET * Bm * (delta[:, ch] * u[:, ch])[:, None]).sum(0)
    Y = TF.silu(z) * y
    F = 0.5 * torch.cat([t(w["beta_attn"]) * TF.rms_norm(O, (H * hd,), eps=dims.eps),
                         t(w["beta_ssm"]) * TF.rms_norm(Y, (D,), eps=dims.eps)], dim=-1)
    out = TF.linear(F, t(w["w_out"]))
    return dict(out=out[m:].numpy(), h=hT.numpy(), K=kk.view(T, G, hd).numpy(),
                xs=xs.numpy(), O=O[m:].numpy(), Y=Y[m:].numpy())


GQA_ROPE = replace(GQA, rope_base=100.0)
GQA_M2 = replace(GQA, ssm_heads=3)                   # Mamba2 heads of 8 channels


@pytest.mark.parametrize("dims,n,window,is_global", [
    (TINY, 40, 16, False), (TINY, 24, 16, True), (GQA, 30, 7, False), (GQA, 17, 5, True),
    (GQA_ROPE, 30, 7, False), (replace(TINY, rope_base=10000.0), 24, 16, True),
    (GQA_M2, 30, 7, False), (replace(TINY, ssm_heads=8), 24, 16, True)])
def test_layer_matches_library_composition(dims, n, window, is_global):
    x, R, w = _layer(dims, n, seed=11)
    got = ref.prefill(dims.as_dict(), w, R, x, window, is_global)
    want = layer_by_library(dims, w, R, x[0], window, is_global)
    np.testing.assert_allclose(got["out"][0], want["out"], rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(got["h"][0], want["h"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["K_all"][0], want["K"], rtol=1e-12, atol=1e-12)
    k = dims.d_conv
    np.testing.assert_allclose(got["conv_tail"][0], want["xs"][-(k - 1):], rtol=1e-12, atol=1e-12)


def test_meta_prefix_matches_prefill_state():
    """The offline meta part equals the state of the literal [R; X] pass at row m."""
    dims = TINY
    x, R, w = _layer(dims, 1, seed=5)
    mp = ref.meta_prefix(dims.as_dict(), w, R)
    want = layer_by_library(dims, w, R, x[0][:0], 16, False)
    np.testing.assert_allclose(mp["h0"], want["h"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(mp["k"].transpose(1, 0, 2), want["K"], rtol=1e-12)
    np.testing.assert_allclose(mp["conv_tail"], want["xs"][-3:], rtol=1e-12)


# ---------------------------------------------------------------------------
# hand-derived golden values
# ---------------------------------------------------------------------------
def test_golden_scan_geometric():
    rows = _golden("scan_geometric.txt")
    T = len(rows)
    ln2 = math.log(2.0)
    y, h = ref.selective_scan(np.ones((T, 1)), np.full((T, 1), ln2),
                              np.array([[-1.0, -2.0]]), np.tile([[1.0, 2.0]], (T, 1)),
                              np.ones((T, 2)), np.zeros((1, 2)))
    for t, (tt, y_ln2, h0, h1) in enumerate(rows):
        assert int(tt) == t
        assert y[t, 0] == pytest.approx(y_ln2 * ln2, rel=1e-14)
    assert h[0, 0] == pytest.approx(rows[-1][2] * ln2, rel=1e-14)
    assert h[0, 1] == pytest.approx(rows[-1][3] * ln2, rel=1e-14)


def test_golden_attention_two_keys():
    (p1, p2), o_want = _golden("attention_two_keys.txt")
    q = np.array([[1.0, 0, 0, 0]])
    K = np.zeros((2, 1, 4)); K[0, 0, 0] = 2 * math.log(3.0)
    V = np.zeros((2, 1, 4)); V[0, 0, 0] = 4.0; V[1, 0, 1] = 8.0
    o, p = ref.attend(q, K, V, np.array([0, 1]), 1.0 / math.sqrt(4))
    np.testing.assert_allclose(p[0], [p1, p2], rtol=1e-14)
    np.testing.assert_allclose(o[0], o_want, rtol=1e-14, atol=1e-14)


def test_golden_conv_taps():
    xs_in, c_want = _golden("conv_taps.txt")
    c = ref.causal_conv(np.array(xs_in)[:, None], np.array([[1.0, 2, 3, 4]]),
                        np.zeros(1), np.zeros((3, 1)))
    np.testing.assert_array_equal(c[:, 0], c_want)


def test_softplus_silu_closed_forms():
    assert ref.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    assert ref.softplus(50.0) == pytest.approx(50.0 + math.exp(-50.0), rel=1e-15)
    assert ref.softplus(-50.0) == pytest.approx(math.exp(-50.0), rel=1e-12)
    assert ref.silu(0.0) == 0.0
    assert ref.silu(2.0) == pytest.approx(2.0 / (1.0 + math.exp(-2.0)), rel=1e-15)
    assert ref.silu(-800.0) == pytest.approx(0.0, abs=1e-300)


# ---------------------------------------------------------------------------
# invariants and special cases
# ---------------------------------------------------------------------------
def test_window_at_least_n_equals_global():
    dims = GQA
    x, R, w = _layer(dims, 20, seed=3)
    a = ref.prefill(dims.as_dict(), w, R, x, 20, False)
    b = ref.prefill(dims.as_dict(), w, R, x, 10 ** 6, False)
    c = ref.prefill(dims.as_dict(), w, R, x, 1, True)
    np.testing.assert_allclose(a["out"], c["out"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(b["out"], c["out"], rtol=1e-13, atol=1e-13)
    d_ = ref.prefill(dims.as_dict(), w, R, x, 19, False)
    assert np.abs(d_["out"] - c["out"]).max() > 1e-6   # the window does bite below n


def test_allowed_rows_shape():
    m, W = 4, 3
    assert list(ref.allowed_rows(m + 0, m, W, False)) == [0, 1, 2, 3, 4]
    assert list(ref.allowed_rows(m + 5, m, W, False)) == [0, 1, 2, 3, 7, 8, 9]
    assert list(ref.allowed_rows(m + 5, m, W, True)) == [0, 1, 2, 3, 4, 5, 6, 7, 8, 9]


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((4, 8)) * 3
    K = rng.standard_normal((30, 2, 8)) * 3
    V = rng.standard_normal((30, 2, 8))
    for i in (3, 10, 29):
        rows = ref.allowed_rows(i, 3, 5, False)
        _, p = ref.attend(q, K, V, rows, 1 / math.sqrt(8))
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-14)
        assert p.shape[1] == 3 + min(5, i - 3 + 1)


def test_quiet_attention_zero_token():
    """A K = V = 0 key adds exactly 1 to the softmax denominator (paper §2.3,
    'exit tokens'): o = sum e^s v / (1 + sum e^s)."""
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 8))
    K = rng.standard_normal((6, 1, 8)); K[0] = 0.0
    V = rng.standard_normal((6, 1, 8)); V[0] = 0.0
    o, _ = ref.attend(q, K, V, np.arange(6), 1.0)
    s = K[1:, 0] @ q[0]
    want = (np.exp(s)[:, None] * V[1:, 0]).sum(0) / (1.0 + np.exp(s).sum())
    np.testing.assert_allclose(o[0], want, rtol=1e-13)


def test_gqa_equals_mha_with_duplicated_heads():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((4, 8))
    K = rng.standard_normal((12, 2, 8))
    V = rng.standard_normal((12, 2, 8))
    rows = np.arange(12)
    o_gqa, _ = ref.attend(q, K, V, rows, 0.3)
    Kd, Vd = np.repeat(K, 2, axis=1), np.repeat(V, 2, axis=1)
    o_mha, _ = ref.attend(q, Kd, Vd, rows, 0.3)
    np.testing.assert_allclose(o_gqa, o_mha, rtol=1e-14)
    # heads 0,1 read group 0 and heads 2,3 read group 1
    o_h2, _ = ref.attend(q[2:3], K[:, 1:2], V[:, 1:2], rows, 0.3)
    np.testing.assert_allclose(o_gqa[2], o_h2[0], rtol=1e-14)


def test_zero_delta_keeps_state():
    rng = np.random.default_rng(4)
    T, D, N = 7, 5, 3
    h0 = rng.standard_normal((D, N))
    Cm = rng.standard_normal((T, N))
    y, h = ref.selective_scan(rng.standard_normal((T, D)), np.zeros((T, D)),
                              -np.exp(rng.standard_normal((D, N))),
                              rng.standard_normal((T, N)), Cm, h0)
    np.testing.assert_array_equal(h, h0)
    np.testing.assert_allclose(y, (h0 @ Cm.T).T, rtol=1e-14)


def test_constant_input_geometric_sum():
    rng = np.random.default_rng(6)
    T, D, N = 50, 4, 3
    A = -np.exp(rng.uniform(0, 2, (D, N)))
    dlt = rng.uniform(0.01, 0.2, D)
    u = rng.standard_normal(D)
    Bv = rng.standard_normal(N)
    h0 = rng.standard_normal((D, N))
    _, h = ref.selective_scan(np.tile(u, (T, 1)), np.tile(dlt, (T, 1)), A,
                              np.tile(Bv, (T, 1)), np.ones((T, N)), h0)
    a = np.exp(dlt[:, None] * A)
    inj = (dlt * u)[:, None] * Bv[None, :]
    want = a ** T * h0 + inj * (1 - a ** T) / (1 - a)
    np.testing.assert_allclose(h, want, rtol=1e-12)


def test_full_decay_limit():
    """A -> -inf: the state forgets everything, h_t = Delta_t u_t B_t."""
    rng = np.random.default_rng(7)
    T, D, N = 6, 3, 4
    dlt = rng.uniform(0.1, 1, (T, D)); u = rng.standard_normal((T, D))
    Bm = rng.standard_normal((T, N)); Cm = rng.standard_normal((T, N))
    y, h = ref.selective_scan(u, dlt, np.full((D, N), -1e300), Bm, Cm,
                              rng.standard_normal((D, N)))
    np.testing.assert_allclose(y, (dlt * u) * (Bm * Cm).sum(1)[:, None], rtol=1e-13)
    np.testing.assert_allclose(h, (dlt[-1] * u[-1])[:, None] * Bm[-1][None, :], rtol=1e-13)


def test_beta_zero_selects_one_branch():
    """beta1 = 0 leaves only 1/2 W_out[:, Wa:] norm(Y); beta2 = 0 only the
    attention half (paper §2.1 and App. C head-importance analysis)."""
    dims = TINY
    x, R, w = _layer(dims, 12, seed=8)
    Wa = dims.attn_width
    full = ref.prefill(dims.as_dict(), w, R, x, 16, False)
    O, Y = full["O"][0], full["Y"][0]
    nrm = lambda v: v / np.sqrt((v * v).mean(-1, keepdims=True) + dims.eps)
    w1 = dict(w, beta_attn=np.zeros_like(w["beta_attn"]))
    got = ref.prefill(dims.as_dict(), w1, R, x, 16, False)["out"][0]
    np.testing.assert_allclose(got, 0.5 * nrm(Y) @ w["w_out"][:, Wa:].T.astype(np.float64),
                               rtol=1e-11, atol=1e-12)
    w2 = dict(w, beta_ssm=np.zeros_like(w["beta_ssm"]))
    got = ref.prefill(dims.as_dict(), w2, R, x, 16, False)["out"][0]
    np.testing.assert_allclose(got, 0.5 * nrm(O) @ w["w_out"][:, :Wa].T.astype(np.float64),
                               rtol=1e-11, atol=1e-12)


def test_consumer_reads_producer_kv():
    """A consumer with the producer's Q weights and input gives the producer's
    attention output; its K/V are the producer's, bit for bit."""
    dims = GQA
    x, R, wp = _layer(dims, 15, seed=9, kv_producer=True)
    rng = np.random.default_rng(9)
    _ = rng  # the consumer draw drops the K/V rows of the same weights
    Wa, kv = dims.attn_width, dims.n_kv_heads * dims.head_dim
    wc = dict(wp, kv_producer=False,
              w_in=np.concatenate([wp["w_in"][:Wa], wp["w_in"][Wa + 2 * kv:]]))
    prod = ref.prefill(dims.as_dict(), wp, R, x, 6, False)
    cons = ref.prefill(dims.as_dict(), wc, R, x, 6, False,
                       shared_kv=(prod["K_all"], prod["V_all"]))
    np.testing.assert_array_equal(cons["K_all"], prod["K_all"])
    np.testing.assert_allclose(cons["O"], prod["O"], rtol=1e-14)
    np.testing.assert_allclose(cons["out"], prod["out"], rtol=1e-13)


@pytest.mark.parametrize("is_global,n0,steps,cap,dims", [
    (False, 5, 4, 6, GQA), (False, 9, 6, 6, GQA), (True, 5, 4, 16, GQA),
    (False, 9, 6, 6, GQA_ROPE), (True, 5, 4, 16, GQA_ROPE), (False, 9, 6, 6, GQA_M2)])
def test_prefill_then_decode_equals_longer_prefill(is_global, n0, steps, cap, dims):
    """prefill(n) + k decode steps == prefill(n + k): outputs, state, conv
    tail and cache slots (including ring wrap-around when n + k > cap); with
    RoPE this also pins the decode token's position to the prefill's."""
    window = cap
    x, R, w = _layer(dims, n0 + steps, seed=10, batch=2)
    B = x.shape[0]
    G, hd = dims.n_kv_heads, dims.head_dim
    zeros = np.zeros((B, G, cap, hd))
    cache0 = dict(k=zeros, v=zeros, is_ring=not is_global)
    full = ref.prefill(dims.as_dict(), w, R, x, window, is_global, cache=cache0)
    pre = ref.prefill(dims.as_dict(), w, R, x[:, :n0], window, is_global, cache=cache0)
    mp = ref.meta_prefix(dims.as_dict(), w, R)
    cache = dict(k=pre["cache_k"], v=pre["cache_v"], len=np.full(B, n0), is_ring=not is_global)
    h, conv = pre["h"], pre["conv_tail"]
    for s in range(steps):
        r = ref.decode_step(dims.as_dict(), w, x[:, n0 + s], mp["k"], mp["v"], window,
                            is_global, cache, h, conv)
        np.testing.assert_allclose(r["out"], full["out"][:, n0 + s], rtol=1e-10, atol=1e-11)
        cache = dict(k=r["cache_k"], v=r["cache_v"], len=r["len"], is_ring=not is_global)
        h, conv = r["h"], r["conv"]
    np.testing.assert_allclose(h, full["h"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(conv, full["conv_tail"], rtol=1e-12)
    # same slots hold the same positions (values agree up to BLAS rounding order)
    np.testing.assert_allclose(cache["k"], full["cache_k"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(cache["v"], full["cache_v"], rtol=1e-12, atol=1e-14)
    assert list(cache["len"]) == [n0 + steps] * B


def test_ring_slot_holds_last_position_with_that_residue():
    dims = GQA
    x, R, w = _layer(dims, 13, seed=12)
    cap = 5
    zeros = np.zeros((1, dims.n_kv_heads, cap, dims.head_dim))
    r = ref.prefill(dims.as_dict(), w, R, x, cap, False,
                    cache=dict(k=zeros, v=zeros, is_ring=True))
    for s in range(cap):
        p = max(q for q in range(13) if q % cap == s)
        np.testing.assert_array_equal(r["cache_k"][0, :, s], r["k_full"][0, :, p])
        np.testing.assert_array_equal(r["cache_v"][0, :, s], r["v_full"][0, :, p])


def test_consumer_decode_sees_token_appended_by_producer():
    dims = GQA
    x, R, wp = _layer(dims, 8, seed=13, batch=2)
    Wa, kv = dims.attn_width, dims.n_kv_heads * dims.head_dim
    wc = dict(wp, kv_producer=False,
              w_in=np.concatenate([wp["w_in"][:Wa], wp["w_in"][Wa + 2 * kv:]]))
    mp = ref.meta_prefix(dims.as_dict(), wp, R)
    cap = 4
    pre = ref.prefill(dims.as_dict(), wp, R, x[:, :7], cap, False,
                      cache=dict(k=np.zeros((2, 2, cap, 8)), v=np.zeros((2, 2, cap, 8)),
                                 is_ring=True))
    cache = dict(k=pre["cache_k"], v=pre["cache_v"], len=np.full(2, 7), is_ring=True)
    rp = ref.decode_step(dims.as_dict(), wp, x[:, 7], mp["k"], mp["v"], cap, False,
                         cache, pre["h"], pre["conv_tail"])
    cache2 = dict(k=rp["cache_k"], v=rp["cache_v"], len=rp["len"], is_ring=True)
    rc = ref.decode_step(dims.as_dict(), wc, x[:, 7], mp["k"], mp["v"], cap, False,
                         cache2, pre["h"], pre["conv_tail"])
    np.testing.assert_allclose(rc["out"], rp["out"], rtol=1e-13)
    np.testing.assert_array_equal(rc["cache_k"], rp["cache_k"])
    assert list(rc["len"]) == [8, 8]


# ---------------------------------------------------------------------------
# the block around the layer (pre-norms, residuals, SiLU-gated MLP)
# ---------------------------------------------------------------------------
def _block(dims: LayerDims, n, seed, d_ff=20, kv_producer=True, batch=1):
    from hybrid_attention_ssm_amd.synth import block_weights
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((batch, n, dims.d_model)).astype(np.float32)
    R = rng.standard_normal((dims.n_meta, dims.d_model)).astype(np.float32)
    return x, R, block_weights(rng, dims, d_ff, kv_producer)


def block_by_library(dims: LayerDims, bw, R, xb, window, is_global, store=None):
    """x1 = x + layer(rms_norm(x; g1)); out = x1 + down(silu(gate) * up) of
    rms_norm(x1; g2), with torch's rms_norm, linear and silu; the gate/up rows
    are taken from the even/odd rows of the stored matrix.  store (optional):
    the rounding a 16-bit path applies to what it hands from one kernel to the
    next: the layer's inputs, the residual x1, the MLP's input and its hidden
    units."""
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    st = (lambda v: t(store(np.asarray(v, dtype=np.float32)))) if store else t
    d = dims.d_model
    n1 = lambda v: st(TF.rms_norm(t(v), (d,), weight=t(bw["norm1"]), eps=dims.eps)).numpy()
    layer = layer_by_library(dims, bw["mixer"], n1(R), n1(xb), window, is_global)
    x1 = st(t(xb) + t(layer["out"]))
    n2 = st(TF.rms_norm(x1, (d,), weight=t(bw["norm2"]), eps=dims.eps))
    w = t(bw["w_gate_up"])
    hidden = st(TF.silu(TF.linear(n2, w[0::2])) * TF.linear(n2, w[1::2]))
    return dict(out=(x1 + TF.linear(hidden, t(bw["w_down"]))).numpy(), x1=x1.numpy(), h=layer["h"])


@pytest.mark.parametrize("dims,n,window,is_global", [(TINY, 21, 8, False), (GQA, 17, 5, True)])
def test_block_matches_library_composition(dims, n, window, is_global):
    x, R, bw = _block(dims, n, seed=31)
    got = ref.block_prefill(dims.as_dict(), bw, R, x, window, is_global)
    want = block_by_library(dims, bw, R, x[0], window, is_global)
    np.testing.assert_allclose(got["out"][0], want["out"], rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(got["x1"][0], want["x1"], rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(got["h"][0], want["h"], rtol=1e-10, atol=1e-12)


def _round_bf16(v):
    from hybrid_attention_ssm_amd.synth import round_bf16
    return round_bf16(v)


@pytest.mark.parametrize("dims,n,window,is_global", [(TINY, 21, 8, False), (GQA, 17, 5, True)])
def test_block_with_stored_operands_matches_library_composition(dims, n, window, is_global):
    """The oracle's `store` hook: rounding at the layer inputs, the residual
    after the layer, the MLP input and the MLP hidden units, against the torch
    composition that rounds at the same four points."""
    x, R, bw = _block(dims, n, seed=35)
    got = ref.block_prefill(dims.as_dict(), bw, R, x, window, is_global, store=_round_bf16)
    want = block_by_library(dims, bw, R, x[0], window, is_global, store=_round_bf16)
    np.testing.assert_allclose(got["out"][0], want["out"], rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(got["x1"][0], want["x1"], rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(got["h"][0], want["h"], rtol=1e-10, atol=1e-12)
    # the rounding is really applied: x1 holds bf16 values, and the result
    # differs from the unrounded block by far more than the fp64 noise
    assert np.array_equal(_round_bf16(got["x1"]).astype(np.float64), got["x1"])
    exact = ref.block_prefill(dims.as_dict(), bw, R, x, window, is_global)
    assert np.abs(exact["out"] - got["out"]).max() > 1e-4


def test_block_decode_with_stored_operands_equals_longer_prefill():
    """store applies per row, so prefill(n0) + decode steps with rounding at
    the same points equals prefill(n0 + k) with it."""
    dims = GQA
    n0, steps, cap = 6, 4, 6
    x, R, bw = _block(dims, n0 + steps, seed=36, batch=2)
    B = x.shape[0]
    zeros = np.zeros((B, dims.n_kv_heads, cap, dims.head_dim))
    cache0 = dict(k=zeros, v=zeros, is_ring=True)
    st = _round_bf16
    full = ref.block_prefill(dims.as_dict(), bw, R, x, cap, False, cache=cache0, store=st)
    pre = ref.block_prefill(dims.as_dict(), bw, R, x[:, :n0], cap, False, cache=cache0, store=st)
    mp = ref.block_meta_prefix(dims.as_dict(), bw, R, store=st)
    cache = dict(k=pre["cache_k"], v=pre["cache_v"], len=np.full(B, n0), is_ring=True)
    h, conv = pre["h"], pre["conv_tail"]
    for s_ in range(steps):
        r = ref.block_decode_step(dims.as_dict(), bw, x[:, n0 + s_], mp["k"], mp["v"], cap,
                                  False, cache, h, conv, store=st)
        np.testing.assert_allclose(r["out"], full["out"][:, n0 + s_], rtol=1e-10, atol=1e-11)
        cache = dict(k=r["cache_k"], v=r["cache_v"], len=r["len"], is_ring=True)
        h, conv = r["h"], r["conv"]
    np.testing.assert_allclose(h, full["h"], rtol=1e-10, atol=1e-12)


def test_rms_norm_closed_form():
    # rms([3, 4]) = sqrt(12.5)
    got = ref.rms_norm(np.array([3.0, 4.0]), np.array([2.0, 1.0]), 0.0)
    r = math.sqrt(12.5)
    np.testing.assert_allclose(got, [6.0 / r, 4.0 / r], rtol=1e-15)


def test_mlp_gate_is_the_even_row():
    """SiLU(v) -> v for large v and -> 0 for very negative v: with the gate on
    coordinate 0 and the up projection on coordinate 1, the output is the
    down column times v0 * v1 or nearly zero, never the other way round."""
    w_gu = np.array([[1.0, 0.0], [0.0, 1.0]])     # row 0 gate = e0, row 1 up = e1
    w_down = np.array([[2.0], [-3.0]])
    big = ref.mlp(np.array([40.0, 0.5]), w_gu, w_down)
    np.testing.assert_allclose(big, [2.0 * 40.0 * 0.5, -3.0 * 40.0 * 0.5], rtol=1e-15)
    tiny = ref.mlp(np.array([-40.0, 0.5]), w_gu, w_down)
    assert np.abs(tiny).max() < 1e-15 * 40 + 1e-15
    swapped = ref.mlp(np.array([0.5, 40.0]), w_gu, w_down)    # gate sees 0.5, up sees 40
    assert abs(swapped[0] - 2.0 * 0.5 / (1.0 + math.exp(-0.5)) * 40.0) < 1e-12


def test_block_is_identity_when_both_branches_are_zero():
    dims = GQA
    x, R, bw = _block(dims, 9, seed=32)
    bw = dict(bw, mixer=dict(bw["mixer"], w_out=np.zeros_like(bw["mixer"]["w_out"])),
              w_down=np.zeros_like(bw["w_down"]))
    got = ref.block_prefill(dims.as_dict(), bw, R, x, 4, False)
    np.testing.assert_array_equal(got["out"], x.astype(np.float64))


def test_block_prefill_then_decode_equals_longer_prefill():
    dims = GQA
    n0, steps, cap = 6, 5, 6
    x, R, bw = _block(dims, n0 + steps, seed=33, batch=2)
    B = x.shape[0]
    zeros = np.zeros((B, dims.n_kv_heads, cap, dims.head_dim))
    cache0 = dict(k=zeros, v=zeros, is_ring=True)
    full = ref.block_prefill(dims.as_dict(), bw, R, x, cap, False, cache=cache0)
    pre = ref.block_prefill(dims.as_dict(), bw, R, x[:, :n0], cap, False, cache=cache0)
    mp = ref.block_meta_prefix(dims.as_dict(), bw, R)
    cache = dict(k=pre["cache_k"], v=pre["cache_v"], len=np.full(B, n0), is_ring=True)
    h, conv = pre["h"], pre["conv_tail"]
    for s in range(steps):
        r = ref.block_decode_step(dims.as_dict(), bw, x[:, n0 + s], mp["k"], mp["v"], cap,
                                  False, cache, h, conv)
        np.testing.assert_allclose(r["out"], full["out"][:, n0 + s], rtol=1e-10, atol=1e-11)
        cache = dict(k=r["cache_k"], v=r["cache_v"], len=r["len"], is_ring=True)
        h, conv = r["h"], r["conv"]
    np.testing.assert_allclose(h, full["h"], rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# rotary position embedding
# ---------------------------------------------------------------------------
def test_rope_equals_complex_multiplication():
    rng = np.random.default_rng(40)
    for hd, base in ((8, 100.0), (64, 10000.0), (32, 500000.0)):
        v = rng.standard_normal((7, 3, hd))
        pos = rng.integers(0, 9000, size=(7, 1))
        want = rope_by_complex(v, pos, base).numpy()
        # angles reach 9000 rad: fp64 sin/cos of them agree to ~1e-12
        np.testing.assert_allclose(ref.rope(v, pos, base), want, rtol=1e-10, atol=1e-10)


def test_rope_is_a_position_linear_rotation():
    rng = np.random.default_rng(41)
    hd, base = 16, 1000.0
    v = rng.standard_normal((5, hd))
    half = hd // 2
    r = ref.rope(v, 37, base)
    # each pair keeps its length; position 0 and base 0 change nothing
    np.testing.assert_allclose(r[:, :half] ** 2 + r[:, half:] ** 2,
                               v[:, :half] ** 2 + v[:, half:] ** 2, rtol=1e-12)
    np.testing.assert_array_equal(ref.rope(v, 0, base), v)
    np.testing.assert_array_equal(ref.rope(v, 37, 0.0), v)
    # turning by p1 then p2 is turning by p1 + p2
    np.testing.assert_allclose(ref.rope(ref.rope(v, 11, base), 26, base), r, rtol=1e-12, atol=1e-12)
    # scores depend on the distance only
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)
    s1 = ref.rope(q, 50, base) @ ref.rope(k, 20, base)
    s2 = ref.rope(q, 1030, base) @ ref.rope(k, 1000, base)
    np.testing.assert_allclose(s1, s2, rtol=1e-10)


def test_meta_prefix_keys_carry_meta_positions():
    x, R, w = _layer(GQA_ROPE, 6, seed=42)
    mp = ref.meta_prefix(GQA_ROPE.as_dict(), w, R)
    pre = ref.prefill(GQA_ROPE.as_dict(), w, R, x, 4, False)
    m = GQA_ROPE.n_meta
    np.testing.assert_allclose(mp["k"], pre["K_all"][0, :m].transpose(1, 0, 2), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Mamba2 SSM heads
# ---------------------------------------------------------------------------
def test_mamba2_heads_of_one_channel_are_mamba_with_state_independent_decay():
    """S = D heads of one channel each: Mamba heads whose A row is one value."""
    dims2 = replace(GQA, ssm_heads=GQA.d_inner)
    x, R, w2 = _layer(dims2, 12, seed=44)
    w1 = dict(w2, A=np.repeat(np.asarray(w2["A"]).reshape(-1, 1), GQA.d_state, axis=1))
    a = ref.prefill(dims2.as_dict(), w2, R, x, 5, False)
    b = ref.prefill(GQA.as_dict(), w1, R, x, 5, False)
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a["h"], b["h"], rtol=1e-12, atol=1e-14)


def test_mamba2_meta_prefix_matches_prefill_state():
    x, R, w = _layer(GQA_M2, 1, seed=45)
    mp = ref.meta_prefix(GQA_M2.as_dict(), w, R)
    # the state after the meta rows is the state a prefill starts its real rows from:
    # a prefill of one real token from zero equals one decode step from mp
    pre = ref.prefill(GQA_M2.as_dict(), w, R, x, 4, False)
    cache = dict(k=np.zeros((1, GQA_M2.n_kv_heads, 4, GQA_M2.head_dim)), v=np.zeros((1, GQA_M2.n_kv_heads, 4, GQA_M2.head_dim)),
                 len=np.zeros(1, np.int64), is_ring=True)
    r = ref.decode_step(GQA_M2.as_dict(), w, x[:, 0], mp["k"], mp["v"], 4, False, cache,
                        mp["h0"][None], mp["conv_tail"][None])
    np.testing.assert_allclose(r["out"], pre["out"][:, 0], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(r["h"], pre["h"], rtol=1e-10, atol=1e-12)
