"""The seeded input generator: determinism, the recipe's transforms and rounding (CPU only)."""
import numpy as np
import pytest
import torch

from complex_valued_attention_amd import inputs as gen
from oracle import born_attention


def test_deterministic_and_seed_dependent():
    a = gen.make_inputs("born_causal_c64_b1h1t128d16")
    b = gen.make_inputs("born_causal_c64_b1h1t128d16")
    c = gen.make_inputs("born_causal_c64_b1h1t128d16", seed=7)
    assert np.array_equal(a.dev["q"], b.dev["q"]) and np.array_equal(a.dev["v"], b.dev["v"])
    assert not np.array_equal(a.dev["q"], c.dev["q"])
    assert a.dev["q"].dtype == np.complex64 and a.dev["q"].shape == (1, 1, 128, 16)


def test_circular_complex_normal_moments():
    q, k, v = gen.random_qkv(2, 2, 4096, 16, seed=1)
    for z in (q, k, v):
        assert abs(np.mean(np.abs(z) ** 2) - 1.0) < 0.02        # E|z|^2 = 1
        assert abs(np.mean(z.real ** 2) - 0.5) < 0.02
        assert abs(np.mean(z * z)) < 0.02                       # E z^2 = 0 (circular)


def test_unit_norm_and_rotary():
    w = gen.WORKLOADS["born_causal_c64_b4h8t1024d64_rotary"]
    q, k, v = gen.random_qkv(1, 2, 256, 64, seed=w.seed, qk_unit=True, v_unit=True, rotary=True)
    for z in (q, k, v):
        np.testing.assert_allclose(np.linalg.norm(z, axis=-1), 1.0, rtol=1e-12)
    # the rotary phase is exp(i t theta_m): undo it and compare with the unrotated draw
    q0, _, _ = gen.random_qkv(1, 2, 256, 64, seed=w.seed, qk_unit=True, v_unit=True, rotary=False)
    theta = 10000.0 ** (-np.arange(64) / 64)
    t = np.arange(256)[:, None]
    np.testing.assert_allclose(q * np.exp(-1j * t * theta), q0, rtol=1e-12, atol=1e-14)


def test_rotary_relative_position_born_weights():
    # the rotary phase makes <q_t, k_s> depend on positions only through t - s:
    # shifting every position by D leaves Born outputs unchanged
    rng = np.random.default_rng(3)
    T, d, D = 40, 8, 17
    q = rng.standard_normal((T, d)) + 1j * rng.standard_normal((T, d))
    k = rng.standard_normal((T, d)) + 1j * rng.standard_normal((T, d))
    v = rng.standard_normal((T, d)) + 1j * rng.standard_normal((T, d))
    theta = 10000.0 ** (-np.arange(d) / d)

    def rot(z, shift):
        t = np.arange(T)[:, None] + shift
        return z * np.exp(1j * t * theta)

    np.testing.assert_allclose(born_attention(rot(q, 0), rot(k, 0), v), born_attention(rot(q, D), rot(k, D), v),
                               rtol=1e-10, atol=1e-12)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(10000) * 10.0 ** rng.integers(-20, 20, 10000),
                        np.array([0.0, -0.0, 1.0, -1.0, 1.00390625, 1.01171875, 3.0e38])])
    bits = gen.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    np.testing.assert_array_equal(gen.bf16_bits_to_f64(bits),
                                  torch.from_numpy(x).to(torch.float32).to(torch.bfloat16).double().numpy())


def test_bf16_workload_layout():
    inp = gen.make_inputs("born_causal_bf16_b8h16t4096d64_rotary", B=1, H=2, T=64)
    for n in ("q_re", "q_im", "k_re", "k_im", "v_re", "v_im"):
        assert inp.dev[n].dtype == np.uint16 and inp.dev[n].shape == (1, 2, 64, 64)
    np.testing.assert_array_equal(inp.q64.real, gen.bf16_bits_to_f64(inp.dev["q_re"]))
    # the oracle reads the rounded values: unit norm holds only to bf16 precision
    assert np.abs(np.linalg.norm(inp.q64, axis=-1) - 1).max() < 1e-2


@pytest.mark.parametrize("name", list(gen.WORKLOADS))
def test_workload_table(name):
    w = gen.WORKLOADS[name]
    assert w.op in ("born", "pct") and w.layout in ("c64", "bf16")
    assert gen.attention_flops(w.T, w.d_h, w.causal, w.B * w.H) > 0


def test_flop_formula():
    # 12 T^2 d_h per head, halved when causal: the bf16 workload is 824.63 GFLOP
    w = gen.WORKLOADS[gen.BENCH_WORKLOAD]
    assert gen.attention_flops(w.T, w.d_h, w.causal, w.B * w.H) == pytest.approx(824.633720832e9)
