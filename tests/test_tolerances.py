"""The parity tests' allowance for bf16 outputs (CPU): half a bf16 ulp of the value,
checked against torch's own round-to-nearest-even conversion to bf16."""
import numpy as np
import torch

from tests.gpu_common import TOL_O_BF16, bf16_half_ulp, o_err


def _to_bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).bfloat16().double().numpy()


def test_half_ulp_bounds_the_bf16_store():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-20, 20, 200000))).astype(np.float32).astype(np.float64)
    assert np.all(np.abs(_to_bf16(x) - x) <= bf16_half_ulp(x))


def test_half_ulp_is_reached_halfway_between_neighbours():
    # each v is a bf16 value; v + half an ulp is exactly representable in fp32 and
    # rounds (to even) to a neighbour exactly half an ulp away
    for v in (1.0, 3.0, 5.5, 2.0 ** -7, 1000.0, -6.25):
        h = float(bf16_half_ulp(v))
        mid = v + h
        assert abs(_to_bf16(mid)[()] - mid) == h, v
    assert bf16_half_ulp(3.0) == 2.0 ** -7 and bf16_half_ulp(1.0) == 2.0 ** -8 and bf16_half_ulp(0.0) == 0.0


def test_o_err_takes_off_only_the_store_rounding():
    rng = np.random.default_rng(1)
    O = rng.uniform(-4.0, 4.0, 4096)
    o = _to_bf16(O)
    assert o_err(o, O, out_bf16=False) > 1e-3  # the store's rounding alone, unforgiven
    assert o_err(o, O, out_bf16=True) <= 1e-6
    bad = o.copy()
    bad[7] += 0.05  # an arithmetic error well past the bar still fails
    assert o_err(bad, O, out_bf16=True) > TOL_O_BF16
    unwritten = o.copy()
    unwritten[5] = np.nan
    assert not o_err(unwritten, O, out_bf16=True) <= TOL_O_BF16
