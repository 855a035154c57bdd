"""Stage-level checks of one prefill: the branch outputs and the fusion.

After an hh_prefill call the workspace still holds what each stage wrote
(offsets from hh_prefill_workspace_layout).

* fp32: the attention branch's O (Hymba paper §2.1 Eq. 1), the SSM branch's
  gated Y (Eq. 2) and the fusion's F = [beta1 norm(O) || beta2 norm(Y)] / 2
  (Eq. 3) against the oracle's O, Y and F of the same call.
* bf16, 1024+ rows: the fused path against the separate norm kernel's path on
  the same inputs.  The fused path stores beta1 * O and beta2 * Y and, in the
  row statistics region, an array [B*n, G] of partial sums of O^2 (one per KV
  group) followed by an array [B*n, ceil(D/64)] of partial sums of Y^2 (one
  per 64-channel block).  Each element of beta * O (beta * Y) must be the
  separate path's O (Y) times beta within two bf16 roundings, and each row's
  partial sums must add up to the sum of squares of that row of O (Y) within
  the rounding of the stored values.  (The bf16 intermediates themselves
  carry the storage precision of their bf16 inputs Q, K, V and z, which the
  oracle does not round; the branch kernels' parity with the oracle on
  controlled inputs is tested through the stage hooks.)
"""
import numpy as np
import pytest
import torch

from hybrid_attention_ssm_amd import binding as hb
from hybrid_attention_ssm_amd.configs import TINY, LayerDims, PrefillWorkload
from hybrid_attention_ssm_amd.synth import prefill_inputs
from oracle import hymba_ref as ref
from tests.harness import TOL, UNIT_ROUNDOFF, np_of, rel_err, run_prefill

pytestmark = pytest.mark.gpu

SMALL_BF16 = LayerDims(d_model=256, n_heads=8, n_kv_heads=2, head_dim=64, d_inner=512,
                       d_state=16, d_conv=4, n_meta=128, dtype="bf16")


def _region(ws: torch.Tensor, off: int, shape, dtype) -> np.ndarray:
    es = torch.empty((), dtype=dtype).element_size()
    n = int(np.prod(shape))
    return np_of(ws[off:off + n * es].view(dtype).view(*shape))


@pytest.mark.parametrize("B,n,W,is_global", [(2, 70, 16, False), (1, 90, 16, True)], ids=["swa", "global"])
def test_prefill_intermediates_match_oracle_f32(B, n, W, is_global):
    dims = TINY
    print(f"case intermediates f32 B={B} n={n} W={W} global={is_global}", flush=True)
    inp = prefill_inputs(PrefillWorkload("mid", 311, dims, B, n, W, is_global), varied=True)
    w = inp["weights"]
    want = ref.prefill(dims.as_dict(), w, inp["R"], inp["x"], W, is_global)
    got = run_prefill(dims, w, inp["R"], inp["x"], W, is_global)
    lay = hb.hh_prefill_workspace_layout(dims, B, n)
    T, Wa, D = B * n, dims.n_heads * dims.head_dim, dims.d_inner
    O = _region(got["ws"], lay["O"], (T, Wa), torch.float32)
    Y = _region(got["ws"], lay["Y"], (T, D), torch.float32)
    F = _region(got["ws"], lay["F"], (T, Wa + D), torch.float32)
    wO, wY = want["O"].reshape(T, Wa), want["Y"].reshape(T, D)
    wF = ref.fuse(wO, wY, w["beta_attn"].astype(np.float64), w["beta_ssm"].astype(np.float64), dims.eps)
    e_o, e_y, e_f = rel_err(O, wO), rel_err(Y, wY), rel_err(F, wF)
    print(f"  err O={e_o:.2e} Y={e_y:.2e} F={e_f:.2e}", flush=True)
    tol = TOL["f32"]
    assert e_o <= tol and e_y <= tol and e_f <= tol


def test_fused_path_intermediates_bf16(monkeypatch):
    dims = SMALL_BF16
    B, n, W = 2, 640, 16
    print(f"case fused intermediates bf16 B={B} n={n} W={W}", flush=True)
    inp = prefill_inputs(PrefillWorkload("midf", 312, dims, B, n, W, False), varied=True)
    w = inp["weights"]
    lay = hb.hh_prefill_workspace_layout(dims, B, n)
    T, Wa, D, G = B * n, dims.n_heads * dims.head_dim, dims.d_inner, dims.n_kv_heads
    gy = (D + 63) // 64
    runs = {}
    for mode in ("0", "1"):
        monkeypatch.setenv("HH_FUSED_NORM", mode)
        got = run_prefill(dims, w, inp["R"], inp["x"], W, False)
        runs[mode] = dict(O=_region(got["ws"], lay["O"], (T, Wa), torch.bfloat16),
                          Y=_region(got["ws"], lay["Y"], (T, D), torch.bfloat16),
                          ssq=_region(got["ws"], lay["SSQ"], (T * (G + gy),), torch.float32))
    sep, fus = runs["0"], runs["1"]
    u = UNIT_ROUNDOFF["bf16"]
    bO, bY = w["beta_attn"].astype(np.float64), w["beta_ssm"].astype(np.float64)
    for name, beta in (("O", bO), ("Y", bY)):
        ref_v = beta * sep[name]
        # the separate path's value is one rounding from the exact one, the fused
        # path's beta * value another: 2u of |beta * value| (+ u^2 terms)
        excess = np.abs(fus[name] - ref_v) - 2.01 * u * np.abs(ref_v)
        print(f"  {name}: max |fused - beta * separate| beyond two roundings = {excess.max():.2e}", flush=True)
        assert excess.max() <= 1e-30
    ssq_o = fus["ssq"][:T * G].reshape(T, G).sum(axis=1)
    ssq_y = fus["ssq"][T * G:].reshape(T, gy).sum(axis=1)
    # sums of squares of the unrounded values against those of the stored ones:
    # each stored value is within u of the exact one, so each square within ~2u
    e_so = np.abs(ssq_o / (sep["O"] ** 2).sum(axis=1) - 1.0).max()
    e_sy = np.abs(ssq_y / (sep["Y"] ** 2).sum(axis=1) - 1.0).max()
    print(f"  row sums of squares: O rel {e_so:.2e}, Y rel {e_sy:.2e}", flush=True)
    assert e_so <= 4 * u and e_sy <= 4 * u
