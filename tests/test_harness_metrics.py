"""The parity metrics themselves (CPU): rel_err_stored allows exactly a
result's own rounding to its storage type and nothing more."""
import numpy as np

from hybrid_attention_ssm_amd.synth import round_bf16
from tests.harness import rel_err, rel_err_stored


def test_storage_rounding_alone_passes():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((257, 129)) * np.exp(rng.uniform(-3, 3, (257, 129)))   # heavy tails
    assert rel_err_stored(round_bf16(x.astype(np.float32)), x, "bf16") == 0.0
    assert rel_err_stored(x.astype(np.float32), x, "f32") == 0.0
    # the plain metric charges the rounding of the largest elements
    assert rel_err(round_bf16(x.astype(np.float32)), x) > 0.0


def test_an_error_beyond_the_rounding_is_measured():
    rng = np.random.default_rng(8)
    x = rng.standard_normal(4096)
    rms = np.sqrt(np.mean(x * x))
    y = round_bf16(x.astype(np.float32)).astype(np.float64)
    i = int(np.argmin(np.abs(x)))          # a near-zero element: its rounding allowance is tiny
    y[i] = x[i] + 0.05 * rms
    assert 0.049 < rel_err_stored(y, x, "bf16") < 0.051
