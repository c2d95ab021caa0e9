"""The seeded input generator: determinism, shapes, bf16 rounding and the step-size recipes."""
import numpy as np
import pytest

from selective_state_space_32_amd import inputs


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 65504.0, 1e-30, -3.0e38],
                                 dtype=np.float32)])
    ours = inputs.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = inputs.bf16_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_ties_round_to_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties go to the even one (1)
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], dtype=np.float32)
    assert list(inputs.bf16_to_f32(inputs.bf16_bits(x))) == [1.0, 1.0 + 2.0 ** -6]


def test_deterministic_and_shapes():
    a = inputs.config_case("c3", L=64, D=128)
    b = inputs.config_case("c3", L=64, D=128)
    assert a.digest() == b.digest()
    assert a.u.shape == (8, 64, 128) and a.u.dtype == np.uint16
    assert a.B.shape == (8, 64, 16) and a.A.shape == (128, 16) and a.A.dtype == np.float32
    assert a.z is not None and a.Dskip.shape == (128,) and a.delta_bias.shape == (128,)
    assert np.all(a.A < 0)
    c = inputs.config_case("c3", L=64, D=128, seed=99)
    assert c.digest() != a.digest()


def test_c1_recipe():
    c = inputs.config_case("c1")
    assert (c.bsz, c.L, c.D, c.N, c.io) == (1, 256, 16, 4, "f32")
    assert np.array_equal(c.A[3], -np.arange(1, 5, dtype=np.float32))
    assert np.all(c.delta_bias == -1.0) and c.z is None
    lti = inputs.config_case("c1_lti")
    assert np.all(lti.delta == lti.delta[:, :1]) and np.all(lti.B == lti.B[:, :1])


def _mean_step(case):
    x = case.values("delta").astype(np.float64) + case.delta_bias.astype(np.float64)
    return float(np.mean(np.logaddexp(0.0, x)))


def test_long_context_mean_step_about_001():
    c = inputs.config_case("c4", L=512)
    assert 0.009 <= _mean_step(c) <= 0.011


def test_layer_step_sizes_in_range():
    c = inputs.config_case("c2", L=256, D=512)
    sp = np.logaddexp(0.0, c.delta_bias.astype(np.float64))
    assert sp.min() >= 0.99e-3 and sp.max() <= 0.1001
    assert 0.04 < _mean_step(c) < 0.075


def test_step_case_recipe():
    s = inputs.step_case(8, 64, 16, 3, seed=5)
    assert s.state0.shape == (8, 64, 16) and s.state0.dtype == np.float32
    assert s.u.shape == (3, 8, 64) and s.B.shape == (3, 8, 16)
    d = s.values("delta")
    assert np.all(d > 0)
    assert 0.05 < float(np.std(s.state0)) < 0.15
