"""CPU oracle for the Hymba hybrid-head layer.

TEST INFRASTRUCTURE ONLY.  Plain, slow, fp64 numpy, written from the Hymba
paper ("Hymba: A Hybrid-head Architecture for Small Language Models", arXiv
2411.13676) and the authors' OpenReview replies to reviewers (same title).
Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import it; the GPU library never calls it and shares no code with it.

Every function computes its definition directly: per-query softmax over
exactly the allowed keys, and the SSM as the literal sequential recurrence.
Library primitives used as steps: matrix products (np.matmul / einsum),
exp, log1p-style softplus, tanh.

Notation: m meta tokens, n real tokens, d model width, H query heads, G KV
heads (query groups), hd head dim, D SSM channels (d_inner), N SSM state,
k conv taps, W window.  X~ = [R; X] has m + n rows; real position p is row
m + p of X~.

Readings where the pages are silent or ambiguous (each is a stated choice):
  * norm = RMSNorm over the whole branch width, eps from dims, no weight of its
    own (beta is the per-channel weight)                  [paper §2.1, Eq. 3]
  * fusion = average: F = 1/2 [beta1*norm(O) || beta2*norm(Y)] followed by one
    output projection W_out [d, H*hd + D]; with equal widths and equal column
    blocks of W_out this is exactly Eq. 3 with the 1/2 of "average"
                                                   [paper §2.1 text; App. B]
  * gate = SiLU(z); conv = causal depthwise conv of k taps with bias, then
    SiLU, applied to the SSM input features only; zero history before the
    first meta token
  * Delta, B, C are linear maps of X~ fused into W_in; Delta = softplus(dt + b)
                                                        [paper §2.1, Eq. 2]
  * discretisation exactly as Eq. 2: decay exp(Delta*A), input Delta*B*u;
    no skip (D) term
  * the window counts real positions only, including the query itself:
    real key j is visible from real query i iff i - W < j <= i; meta rows are
    always visible (the "A-shape" mask of the authors' reply on
    implementation details); global layers see every real j <= i
  * scores are scaled by 1/sqrt(hd)            [authors' reply on Eq. 1 scale]
  * query head h reads KV head floor(h / (H/G))
  * a KV-sharing consumer layer has no K/V projection rows and attends over
    its producer's K/V                   [authors' reply, cache optimisation]
  * rotary position embedding (optional; the pages train with RoPE and change
    its base for the 8k stage, giving neither the base nor the convention):
    with dims["rope_base"] = b > 0, Q and K are rotated after the projection
    and before attention and caching, in the rotate-half pairing: dims i and
    i + hd/2 of a head form pair i, turned by the angle pos * b^(-2i/hd).
    pos is the row of X~ = [R; X], so meta row j sits at position j and real
    position p at m + p; a decode token at real position p is at m + p.
    b = 0 (the default) leaves Q and K as projected.   [paper §3 training]
  * Mamba2 SSM heads (optional; the authors' reply on Mamba vs Mamba2 says
    the hybrid head works with either and reports a model trained with
    Mamba2 heads, without their shapes): with dims["ssm_heads"] = S > 0 the
    D channels form S heads of P = D / S consecutive channels; the dt block
    of the projection has S columns, so Delta_t is per head, and A is one
    negative scalar per head.  The recurrence is Eq. 2 with those shared:
    h_t[c,s] = exp(Delta_t[h] A[h]) h_{t-1}[c,s] + Delta_t[h] u_t[c] B_t[s],
    h = c // P (Mamba-2's scalar-times-identity state matrix).  Everything
    else (conv on xs, SiLU gate, no skip term, B and C shared by all
    channels) is as for the Mamba heads.  S = 0 (the default): Mamba.

The block around the layer (the pages name its MLP width, 5504 at 1.5B in the
architecture table, and draw it in their architecture figure, but do not
write it out; these are the plain pre-norm readings):
  * x1 = x + layer(g1 * norm(x)),  out = x1 + MLP(g2 * norm(x1)), with norm the
    RMS normalisation above and g1, g2 learned per-channel gains; the meta
    rows enter the layer as g1 * norm(R)
  * MLP(v) = W_down (SiLU(W_gate v) * (W_up v)); W_gate and W_up are stored
    as one matrix whose rows alternate gate, up (row 2i gate i, 2i+1 up i)
The block functions take an optional `store` map (default: none).  A path
that keeps its activations in a 16-bit type rounds the values it hands from
one kernel to the next (the layer and MLP inputs, the residual after the
layer, the MLP hidden units) and feeds the rounded values to bf16 matrix
units; passing that rounding as `store` gives the exact result of the same
computation on those stored values.  The arithmetic itself is unchanged.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------------------
# elementwise functions
# ---------------------------------------------------------------------------
def softplus(v):
    """log(1 + exp(v)), evaluated without overflow."""
    return np.logaddexp(0.0, v)


def sigmoid(v):
    return 0.5 * (1.0 + np.tanh(0.5 * v))


def silu(v):
    return v * sigmoid(v)


def _f64(a):
    return np.asarray(a, dtype=F64)


def _dims(dims):
    g = dict(dims)
    return (g["d_model"], g["n_heads"], g["n_kv_heads"], g["head_dim"],
            g["d_inner"], g["d_state"], g["d_conv"], g["n_meta"], g["eps"])


def _rope_base(dims):
    return float(dict(dims).get("rope_base", 0.0) or 0.0)


def _ssm_heads(dims):
    return int(dict(dims).get("ssm_heads", 0) or 0)


def ssm_params(delta, A, dims):
    """Per-channel Delta [..., D] and per-(channel, state) A [D, N] of the SSM
    heads: unchanged for Mamba heads; for Mamba2 heads (header reading) each
    head's Delta and scalar A are shared by its P = D / S channels and A by
    every state."""
    S = _ssm_heads(dims)
    if not S:
        return _f64(delta), _f64(A)
    g = dict(dims)
    D, N = g["d_inner"], g["d_state"]
    P = D // S
    delta_c = np.repeat(_f64(delta), P, axis=-1)
    A_c = np.repeat(np.repeat(_f64(A).reshape(S, 1), P, axis=0), N, axis=1)
    return delta_c, A_c


# ---------------------------------------------------------------------------
# rotary position embedding (header reading: rotate-half pairs, positions are
# the rows of X~)
# ---------------------------------------------------------------------------
def rope(v, pos, base):
    """Rotate the last axis of v [..., hd] for positions pos (shape v.shape[:-1]
    or broadcastable to it).  Pair i = (v[..., i], v[..., i + hd/2]) turns by
    pos * base^(-2i/hd): (a, b) -> (a cos t - b sin t, b cos t + a sin t).
    base 0: v unchanged."""
    v = _f64(v)
    if not base:
        return v.copy()
    hd = v.shape[-1]
    half = hd // 2
    inv_freq = base ** (-2.0 * np.arange(half, dtype=F64) / hd)
    t = np.asarray(pos, dtype=F64)[..., None] * inv_freq
    a, b = v[..., :half], v[..., half:]
    c, s = np.cos(t), np.sin(t)
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# ---------------------------------------------------------------------------
# input projection  [paper §2.1: W_in_proj = [W^Q, W^K, W^V, W^SSM, W^G]]
# ---------------------------------------------------------------------------
def split_projection(P, dims, kv_producer=True):
    """Split the fused projection P = X~ W_in^T into its column blocks.

    Block order: Q (H*hd) | K (G*hd) | V (G*hd) | xs (D) | z (D) | dt (D) |
    B (N) | C (N).  K and V are absent for a KV-sharing consumer layer.
    """
    d, H, G, hd, D, N, k, m, eps = _dims(dims)
    names = ["q"] + (["k", "v"] if kv_producer else []) + ["xs", "z", "dt", "B", "C"]
    dtw = _ssm_heads(dims) or D                 # Delta per head (Mamba2) or per channel
    sizes = [H * hd] + ([G * hd, G * hd] if kv_producer else []) + [D, D, dtw, N, N]
    if P.shape[-1] != sum(sizes):
        raise ValueError(f"projection width {P.shape[-1]} != {sum(sizes)}")
    parts, c = {}, 0
    for name, s in zip(names, sizes):
        parts[name] = P[..., c:c + s]
        c += s
    return parts


# ---------------------------------------------------------------------------
# attention heads  [paper §2.1 Eq. 1; authors' replies: 1/sqrt(d) scale,
# A-shape mask; §2.2 sliding window / global; Table 11 query groups]
# ---------------------------------------------------------------------------
def allowed_rows(i, m, window, is_global):
    """Rows of X~ that real query row i (i >= m) may attend to."""
    lo = m if is_global else max(m, i - window + 1)
    return np.concatenate([np.arange(m), np.arange(lo, i + 1)]).astype(np.int64)


def attend(q, K, V, rows, scale):
    """Softmax attention of one query row over exactly the given key rows.

    q [H, hd]; K, V [R, G, hd]; rows: indices into K/V.
    Returns (o [H, hd], p [H, len(rows)]) with p the softmax weights.
    """
    H, G = q.shape[0], K.shape[1]
    grp = np.arange(H) // (H // G)
    Ks = K[rows][:, grp, :]                      # [L, H, hd]
    Vs = V[rows][:, grp, :]
    s = np.einsum("hd,lhd->hl", q, Ks) * scale   # [H, L]
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    o = np.einsum("hl,lhd->hd", p, Vs)
    return o, p


# ---------------------------------------------------------------------------
# SSM heads  [paper §2.1 Eq. 2 (Mamba selective scan) + the gate G]
# ---------------------------------------------------------------------------
def causal_conv(xs, conv_w, conv_b, history):
    """Depthwise causal conv: c_i = b + sum_{tau<k} w[:, k-1-tau] * xs_{i-tau}.

    xs [T, D]; history [k-1, D] holds the k-1 rows before xs[0] (oldest first).
    """
    k = conv_w.shape[1]
    T = xs.shape[0]
    ext = np.concatenate([history, xs])          # xs[i] == ext[i + k - 1]
    c = np.broadcast_to(conv_b, xs.shape).copy()
    for tau in range(k):
        c += conv_w[:, k - 1 - tau] * ext[k - 1 - tau:k - 1 - tau + T]
    return c


def selective_scan(u, delta, A, Bm, Cm, h):
    """The literal recurrence, one row at a time.

    h_t = exp(delta_t * A) * h_{t-1} + (delta_t * u_t) outer B_t
    y_t = h_t . C_t
    u, delta [T, D]; A [D, N]; Bm, Cm [T, N]; h [D, N] initial state.
    Returns (y [T, D], final h [D, N]).
    """
    T, D = u.shape
    y = np.empty((T, D))
    h = np.array(h, dtype=F64, copy=True)
    decay = np.empty_like(h)
    inject = np.empty_like(h)
    for t in range(T):
        # the same arithmetic as h = exp(delta_t A) h + (delta_t u_t) B_t,
        # written into reused buffers
        np.multiply(delta[t][:, None], A, out=decay)
        np.exp(decay, out=decay)
        np.multiply(decay, h, out=h)
        np.multiply((delta[t] * u[t])[:, None], Bm[t][None, :], out=inject)
        np.add(h, inject, out=h)
        np.dot(h, Cm[t], out=y[t])
    return y, h


# ---------------------------------------------------------------------------
# fusion and output projection  [paper §2.1 Eq. 3; App. B mean fusion]
# ---------------------------------------------------------------------------
def rms_normalize(v, eps):
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)


def fuse(O, Y, beta_attn, beta_ssm, eps):
    """F = 1/2 [beta1 * norm(O) || beta2 * norm(Y)] (row-wise)."""
    return 0.5 * np.concatenate([beta_attn * rms_normalize(O, eps),
                                 beta_ssm * rms_normalize(Y, eps)], axis=-1)


def _weights64(weights):
    w = {k: (_f64(v) if isinstance(v, np.ndarray) else v) for k, v in weights.items()}
    w["kv_producer"] = bool(weights.get("kv_producer", True))
    return w


def _tail(rows, k):
    """Last k-1 rows of `rows` (zero rows in front if there are fewer)."""
    T, D = rows.shape
    t = np.zeros((k - 1, D))
    take = min(T, k - 1)
    if take:
        t[k - 1 - take:] = rows[T - take:]
    return t


# ---------------------------------------------------------------------------
# whole layer, prefill over X~ = [R; X]  [paper §2.3 Eq. 4]
# ---------------------------------------------------------------------------
def prefill(dims, weights, R, x, window, is_global, shared_kv=None, cache=None,
            rows=None):
    """One hybrid-head layer over the prompt x with meta tokens R prepended.

    R [m, d]; x [B, n, d].  shared_kv: for a consumer layer, the producer's
    (K, V) over all m + n rows of X~, each [B, m + n, G, hd].  cache: optional
    dict(k [B, G, cap, hd], v, is_ring) holding the cache contents before the
    call; a producer writes real position p to slot p mod cap (ring) or p.
    rows: real positions whose outputs are wanted (default: all).

    Returns a dict: out [B, len(rows), d]; K_all/V_all [B, m+n, G, hd];
    k_full/v_full [B, G, n, hd] (real rows); h [B, D, N] after the last row;
    conv_tail [B, k-1, D] (xs of the last k-1 rows of X~); cache_k/cache_v
    (if a cache was given); and the branch outputs O, Y for the wanted rows.
    """
    d, H, G, hd, D, N, k, m, eps = _dims(dims)
    w = _weights64(weights)
    R, x = _f64(R), _f64(x)
    Bsz, n, _ = x.shape
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    scale = 1.0 / np.sqrt(hd)
    rope_base = _rope_base(dims)
    out = np.empty((Bsz, len(rows), d))
    K_all = np.empty((Bsz, m + n, G, hd))
    V_all = np.empty((Bsz, m + n, G, hd))
    h_out = np.empty((Bsz, D, N))
    tail_out = np.empty((Bsz, k - 1, D))
    O_all = np.empty((Bsz, len(rows), H * hd))
    Y_all = np.empty((Bsz, len(rows), D))
    for b in range(Bsz):
        Xt = np.concatenate([R, x[b]])                       # X~ = [R, X]
        parts = split_projection(Xt @ w["w_in"].T, dims, w["kv_producer"])
        pos = np.arange(m + n)[:, None]                      # row of X~
        Q = rope(parts["q"].reshape(m + n, H, hd), pos, rope_base)
        if w["kv_producer"]:
            K = rope(parts["k"].reshape(m + n, G, hd), pos, rope_base)
            V = parts["v"].reshape(m + n, G, hd)
        else:
            K, V = _f64(shared_kv[0][b]), _f64(shared_kv[1][b])
        K_all[b], V_all[b] = K, V
        O = np.empty((len(rows), H * hd))
        for r, p in enumerate(rows):
            i = m + int(p)
            o, _ = attend(Q[i], K, V, allowed_rows(i, m, window, is_global), scale)
            O[r] = o.reshape(-1)
        delta, A = ssm_params(softplus(parts["dt"] + w["dt_bias"]), w["A"], dims)
        xs = parts["xs"]
        u = silu(causal_conv(xs, w["conv_w"], w["conv_b"], np.zeros((k - 1, D))))
        y, h = selective_scan(u, delta, A, parts["B"], parts["C"], np.zeros((D, N)))
        Y = y * silu(parts["z"])
        Yr = Y[m + rows]
        F = fuse(O, Yr, w["beta_attn"], w["beta_ssm"], eps)
        out[b] = F @ w["w_out"].T
        h_out[b] = h
        tail_out[b] = _tail(xs, k)
        O_all[b], Y_all[b] = O, Yr
    res = dict(out=out, K_all=K_all, V_all=V_all,
               k_full=K_all[:, m:].transpose(0, 2, 1, 3).copy(),
               v_full=V_all[:, m:].transpose(0, 2, 1, 3).copy(),
               h=h_out, conv_tail=tail_out, O=O_all, Y=Y_all)
    if cache is not None:
        ck, cv = _f64(cache["k"]).copy(), _f64(cache["v"]).copy()
        if w["kv_producer"]:
            cap = ck.shape[2]
            first = max(0, n - cap) if cache["is_ring"] else 0
            last = n if cache["is_ring"] else min(n, cap)
            for p in range(first, last):
                slot = p % cap if cache["is_ring"] else p
                ck[:, :, slot] = K_all[:, m + p]
                cv[:, :, slot] = V_all[:, m + p]
        res["cache_k"], res["cache_v"] = ck, cv
    return res


def meta_prefix(dims, weights, R):
    """What a layer computes from the meta tokens alone, once, offline.

    [paper §2.3: meta tokens are fixed, so their part of the computation can
    be done offline and kept as a learned cache/state initialisation]
    Returns meta K/V [G, m, hd] (producer layers), the SSM state after the m
    meta rows h0 [D, N], and the conv tail [k-1, D] (xs of the last meta rows).
    """
    d, H, G, hd, D, N, k, m, eps = _dims(dims)
    w = _weights64(weights)
    R = _f64(R)
    parts = split_projection(R @ w["w_in"].T, dims, w["kv_producer"])
    res = {}
    if w["kv_producer"]:
        k_rot = rope(parts["k"].reshape(m, G, hd), np.arange(m)[:, None], _rope_base(dims))
        res["k"] = k_rot.transpose(1, 0, 2).copy()
        res["v"] = parts["v"].reshape(m, G, hd).transpose(1, 0, 2).copy()
    delta, A = ssm_params(softplus(parts["dt"] + w["dt_bias"]), w["A"], dims)
    u = silu(causal_conv(parts["xs"], w["conv_w"], w["conv_b"], np.zeros((k - 1, D))))
    _, h = selective_scan(u, delta, A, parts["B"], parts["C"], np.zeros((D, N)))
    res["h0"] = h
    res["conv_tail"] = _tail(parts["xs"], k)
    return res


# ---------------------------------------------------------------------------
# one-token decode step  [authors' replies: KV-sharing groups, meta K/V
# precomputed and pinned; paper §2.2 sliding window / global attention]
# ---------------------------------------------------------------------------
def decode_step(dims, weights, x_t, meta_k, meta_v, window, is_global, cache, h,
                conv, seqs=None):
    """One new token per sequence through one layer.

    x_t [B, d]; meta_k/meta_v [G, m, hd] (shared by all sequences);
    cache: dict(k [B, G, cap, hd], v, len [B] int, is_ring); h [B, D, N];
    conv [B, k-1, D] (xs of the previous k-1 positions, oldest first).
    A producer layer places the token at real position p = len[b], stores its
    K/V in slot p mod cap (ring) or p, and counts it (len + 1).  A consumer
    layer reads the same cache, where its producer has just appended
    position p = len[b] - 1, and writes nothing.  Attention runs over all
    meta keys and the real positions max(0, p - W + 1)..p (global: 0..p).
    seqs: which sequences to compute (default all).
    Returns dict(out [S, d], cache_k, cache_v, len, h [S, D, N], conv [S, k-1, D])
    with cache arrays covering all B sequences (only `seqs` updated).
    """
    d, H, G, hd, D, N, k, m, eps = _dims(dims)
    w = _weights64(weights)
    x_t = _f64(x_t)
    Bsz = x_t.shape[0]
    seqs = np.arange(Bsz) if seqs is None else np.asarray(seqs, dtype=np.int64)
    ck, cv = _f64(cache["k"]).copy(), _f64(cache["v"]).copy()
    length = np.array(cache["len"], dtype=np.int64).copy()
    cap, ring = ck.shape[2], bool(cache["is_ring"])
    mk = _f64(meta_k).transpose(1, 0, 2)                     # [m, G, hd]
    mv = _f64(meta_v).transpose(1, 0, 2)
    scale = 1.0 / np.sqrt(hd)
    out = np.empty((len(seqs), d))
    h_new = np.empty((len(seqs), D, N))
    conv_new = np.empty((len(seqs), k - 1, D))
    rope_base = _rope_base(dims)
    for r, b in enumerate(seqs):
        parts = split_projection(x_t[b] @ w["w_in"].T, dims, w["kv_producer"])
        p = int(length[b]) if w["kv_producer"] else int(length[b]) - 1
        if w["kv_producer"]:
            slot = p % cap if ring else p
            ck[b, :, slot] = rope(parts["k"].reshape(G, hd), m + p, rope_base)
            cv[b, :, slot] = parts["v"].reshape(G, hd)
        lo = 0 if is_global else max(0, p - window + 1)
        slots = [(q % cap if ring else q) for q in range(lo, p + 1)]
        K = np.concatenate([mk, ck[b][:, slots].transpose(1, 0, 2)])   # [m+L, G, hd]
        V = np.concatenate([mv, cv[b][:, slots].transpose(1, 0, 2)])
        q = rope(parts["q"].reshape(H, hd), m + p, rope_base)
        o, _ = attend(q, K, V, np.arange(K.shape[0]), scale)
        win = np.concatenate([_f64(conv[b]), parts["xs"][None, :]])   # [k, D]
        c = _f64(w["conv_b"]) + np.sum(w["conv_w"].T * win, axis=0)
        u = silu(c)
        delta, A = ssm_params(softplus(parts["dt"] + w["dt_bias"]), w["A"], dims)
        hb = np.exp(delta[:, None] * A) * _f64(h[b]) + (delta * u)[:, None] * parts["B"][None, :]
        y = hb @ parts["C"]
        Y = y * silu(parts["z"])
        F = fuse(o.reshape(-1), Y, w["beta_attn"], w["beta_ssm"], eps)
        out[r] = w["w_out"] @ F
        h_new[r] = hb
        conv_new[r] = win[1:]
    if w["kv_producer"]:
        length[seqs] += 1
    return dict(out=out, cache_k=ck, cache_v=cv, len=length, h=h_new, conv=conv_new)


# ---------------------------------------------------------------------------
# the block around the layer: pre-norms, residuals, SiLU-gated MLP
# [architecture table (MLP hidden width) and figure; readings in the header]
# ---------------------------------------------------------------------------
def rms_norm(v, g, eps):
    """g * v / sqrt(mean(v^2) + eps), row-wise."""
    return _f64(g) * rms_normalize(_f64(v), eps)


def _ident(v):
    return v


def mlp(v, w_gate_up, w_down, store=_ident):
    """W_down (SiLU(W_gate v) * W_up v); rows of w_gate_up alternate gate, up."""
    gu = _f64(v) @ _f64(w_gate_up).T
    return _f64(store(silu(gu[..., 0::2]) * gu[..., 1::2])) @ _f64(w_down).T


def block_meta_prefix(dims, bw, R, store=_ident):
    """meta_prefix of the block's layer, whose meta rows are g1 * norm(R)."""
    eps = dict(dims)["eps"]
    return meta_prefix(dims, bw["mixer"], store(rms_norm(R, bw["norm1"], eps)))


def block_prefill(dims, bw, R, x, window, is_global, shared_kv=None, cache=None, store=_ident):
    """One block over the prompt x [B, n, d] with meta rows R [m, d].

    Returns prefill()'s dict for the layer (K/V, state, caches) with `out`
    replaced by the block output and `x1` the residual stream after the layer.
    """
    eps = dict(dims)["eps"]
    x = _f64(x)
    layer = prefill(dims, bw["mixer"], store(rms_norm(R, bw["norm1"], eps)),
                    store(rms_norm(x, bw["norm1"], eps)), window, is_global,
                    shared_kv=shared_kv, cache=cache)
    x1 = _f64(store(x + layer["out"]))
    res = dict(layer)
    res["x1"] = x1
    res["out"] = x1 + mlp(store(rms_norm(x1, bw["norm2"], eps)), bw["w_gate_up"], bw["w_down"], store)
    return res


def block_decode_step(dims, bw, x_t, meta_k, meta_v, window, is_global, cache, h, conv,
                      seqs=None, store=_ident):
    """One new token per sequence through one block (see decode_step)."""
    eps = dict(dims)["eps"]
    x_t = _f64(x_t)
    seqs = np.arange(x_t.shape[0]) if seqs is None else np.asarray(seqs, dtype=np.int64)
    layer = decode_step(dims, bw["mixer"], store(rms_norm(x_t, bw["norm1"], eps)), meta_k, meta_v,
                        window, is_global, cache, h, conv, seqs=seqs)
    x1 = _f64(store(x_t[seqs] + layer["out"]))
    res = dict(layer)
    res["out"] = x1 + mlp(store(rms_norm(x1, bw["norm2"], eps)), bw["w_gate_up"], bw["w_down"], store)
    return res

