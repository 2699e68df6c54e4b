"""CPU checks of the parity tests' error measures (no GPU)."""
import numpy as np

from oracle import moe_oracle as O
from tests.gpu_util import err_beyond_bf16_output, rel_rms_err


def test_err_beyond_bf16_output_is_zero_for_correctly_rounded_outputs():
    rng = np.random.default_rng(1)
    want = rng.standard_normal(20000) * np.exp(2 * rng.standard_normal(20000))
    want[:10] = 0.0
    want[10:20] = rng.standard_normal(10) * 1e-39      # bf16 subnormals
    got = O.bf16_round(want)
    assert rel_rms_err(got, want)[0] > 0               # the rounding itself is visible
    assert err_beyond_bf16_output(got, want) == 0.0


def test_err_beyond_bf16_output_sees_arithmetic_error():
    rng = np.random.default_rng(2)
    want = rng.standard_normal(20000)
    # one output off by 3 % of the RMS before rounding
    s = want.copy()
    s[123] += 0.03 * np.sqrt(np.mean(want ** 2))
    got = O.bf16_round(s)
    e = err_beyond_bf16_output(got, want)
    assert 0.02 < e <= 0.03
    # an output whose exact value lies a quarter ulp (2^-9 at 1.0) from it
    # is within its own rounding
    assert err_beyond_bf16_output(np.array([1.0]), np.array([1.0 + 2.0 ** -9])) == 0.0
