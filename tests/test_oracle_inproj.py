"""Pins of the oracle's affine 4-bit in-projection (oracle/inproj.py).

Each pin fixes one part of the definition independently of the oracle's own
vectorised formula: the order of codes in a word, the group an input belongs
to, the roles of scale and bias, the orientation of the product, and the split
of the output features into qkv, a and b."""
import numpy as np
import pytest
import torch

import oracle
from verify_causal_conv1d_amd import inputs as gi

inproj = oracle.inproj


def _bits(t: torch.Tensor) -> np.ndarray:
    return gi.bf16_bits(t)


def _bf16(values) -> torch.Tensor:
    return torch.tensor(np.asarray(values, np.float32)).to(torch.bfloat16)


def test_code_order_in_a_word():
    w = np.array([[0x76543210, 0xFEDCBA98]], np.uint32).view(np.int32)
    assert inproj.unpack_codes(w, 16).tolist() == [list(range(16))]


@pytest.mark.parametrize("n,k", [(0, 0), (2, 13), (3, 63)])
def test_one_code_selects_one_input(n, k):
    """Scale 1, bias 0 and a single code c at (n, k): column n of y is c x[:, k]
    and every other column is 0, exactly."""
    N, K, G = 4, 64, 32
    codes = np.zeros((N, K), np.int64)
    codes[n, k] = 11
    wq = gi.pack_codes(codes)
    ones = _bits(_bf16(np.ones((N, K // G))))
    zeros = _bits(_bf16(np.zeros((N, K // G))))
    x = _bf16(np.random.default_rng(1).standard_normal((3, K)))
    y = inproj.project(_bits(x), wq, ones, zeros, G)
    ref = np.zeros((3, N))
    ref[:, n] = 11.0 * x.float().numpy().astype(np.float64)[:, k]
    assert np.array_equal(y, ref)


def test_zero_codes_leave_bias_times_group_sums():
    """Codes 0: y[r][n] = sum_g b[n][g] * (sum of x[r] over group g)."""
    rng = np.random.default_rng(2)
    N, K, G = 5, 256, 64
    wq = gi.pack_codes(np.zeros((N, K), np.int64))
    scale = _bits(_bf16(rng.uniform(0.5, 2.0, (N, K // G))))
    bias_t = _bf16(rng.standard_normal((N, K // G)))
    x_t = _bf16(rng.standard_normal((3, K)))
    y = inproj.project(_bits(x_t), wq, scale, _bits(bias_t), G)
    gs = x_t.float().numpy().astype(np.float64).reshape(3, K // G, G).sum(axis=2)
    ref = gs @ bias_t.float().numpy().astype(np.float64).T
    assert np.allclose(y, ref, rtol=1e-14, atol=1e-14)


def test_integer_weights_give_the_exact_integer_product():
    """Scale 1, bias 0, small integer inputs: y is the integer matrix product."""
    rng = np.random.default_rng(3)
    N, K, G = 6, 128, 32
    codes = rng.integers(0, 16, (N, K))
    xi = rng.integers(-8, 9, (4, K))
    ones = _bits(_bf16(np.ones((N, K // G))))
    zeros = _bits(_bf16(np.zeros((N, K // G))))
    y = inproj.project(_bits(_bf16(xi)), gi.pack_codes(codes), ones, zeros, G)
    assert np.array_equal(y, (xi @ codes.T).astype(np.float64))


def test_brute_force_on_a_tiny_projection():
    """Per-element loops over the definition, with a different scale and bias
    per group (powers of two and odd values), against the vectorised oracle."""
    rng = np.random.default_rng(4)
    N, K, G = 3, 64, 32
    codes = rng.integers(0, 16, (N, K))
    s = _bf16(rng.choice([0.25, 0.5, 3.0, -1.5], (N, K // G)))
    b = _bf16(rng.choice([-2.0, 0.125, 5.0], (N, K // G)))
    x = _bf16(rng.standard_normal((2, K)))
    y = inproj.project(_bits(x), gi.pack_codes(codes), _bits(s), _bits(b), G)
    xf, sf, bf = (t.float().numpy().tolist() for t in (x, s, b))
    for r in range(2):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += xf[r][k] * (sf[n][k // G] * codes[n][k] + bf[n][k // G])
            assert abs(acc - y[r, n]) <= 1e-12 * max(1.0, abs(acc))


def test_features_split_into_qkv_a_b():
    shape = gi.Shape(hk=1, hv=2, dk=4, dv=4)
    C = shape.channels
    y = np.arange(3 * (C + 4), dtype=np.float64).reshape(3, C + 4)
    qkv, a, b = inproj.split(y, C, shape.hv)
    assert qkv.shape == (3, C) and a.shape == (3, 2) and b.shape == (3, 2)
    assert np.array_equal(a, y[:, C:C + 2]) and np.array_equal(b, y[:, C + 2:])


def test_synthetic_projection_has_unit_scale_outputs():
    """The synthetic weights give outputs near N(0, 1), the mixer's input
    distribution."""
    t = gi.make_inproj(gi.SMALL, 64, 512, 64, seed=5)
    y = inproj.project(_bits(t.x), t.wq.numpy(), _bits(t.scales), _bits(t.biases), t.group)
    assert 0.6 < y.std() < 1.6 and abs(y.mean()) < 0.2
