"""Pins for the oracle's RMSNorm + 3D RoPE (oracle.norm_rope) and its bf16 rounding.

The pages only say that 3D RoPE and RMSNorm run as fused kernels; the operation they define
here is a reading (RMSNorm over a token's H*D channels, then an axial rotation of adjacent
channel pairs in each head). Each pin checks the oracle against something other than its
own formula: torch's RMSNorm where the rotation is the identity, closed-form rotations of a
single channel pair (as complex multiplications), norm and relative-position invariants of
rotations, and an independent integer implementation of bf16 rounding.
"""
import cmath
import math

import numpy as np
import pytest
import torch

import gen
import oracle


def rand_proj(B, S, H, D, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return gen.f32_to_bf16_bits((rng.standard_normal((B, S, H, D)) * scale).astype(np.float32))


def ones(C):
    return np.full(C, 0x3F80, dtype=np.uint16)  # bf16 1.0


def segments(D):
    f = D // 6
    return [(0, D - 4 * f), (D - 4 * f, 2 * f), (D - 2 * f, 2 * f)]  # (start, size) per axis


def test_round_bf16_agrees_with_integer_rounding_of_float32():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=4000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) < 3.0e38)]
    want = gen.f32_to_bf16_bits(vals)
    got = np.array([oracle.round_bf16(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_round_bf16_ties_and_single_rounding():
    assert oracle.round_bf16(1.0) == 0x3F80
    assert oracle.round_bf16(1.0 + 2.0**-8) == 0x3F80          # tie, even wins
    assert oracle.round_bf16(1.0 + 3 * 2.0**-8) == 0x3F82      # tie, even wins
    assert oracle.round_bf16(-(1.0 + 3 * 2.0**-8)) == 0xBF82
    # just above a tie: a detour through float32 would round to the tie and then down
    assert oracle.round_bf16(1.0 + 2.0**-8 + 2.0**-40) == 0x3F81
    assert oracle.round_bf16(2.0**-133) == 0x0001                # smallest subnormal
    assert oracle.round_bf16(1.4 * 2.0**-133) == 0x0001
    assert oracle.round_bf16(0.0) == 0x0000 and oracle.round_bf16(-0.0) == 0x8000


@pytest.mark.parametrize("D", [64, 128])
def test_position_zero_is_torch_rms_norm(D):
    B, H, grid = 2, 3, (2, 2, 3)
    S = 12
    x = rand_proj(B, S, H, D, 2)
    rng = np.random.default_rng(3)
    w = gen.f32_to_bf16_bits((1.0 + 0.3 * rng.standard_normal(H * D)).astype(np.float32))
    y, _ = oracle.norm_rope(x, w, grid, eps=1e-6)
    xt = torch.from_numpy(gen.bf16_bits_to_f32(x).astype(np.float64)).reshape(B, S, H * D)
    wt = torch.from_numpy(gen.bf16_bits_to_f32(w).astype(np.float64))
    ref = torch.nn.functional.rms_norm(xt, (H * D,), wt, eps=1e-6).numpy().reshape(B, S, H, D)
    # token 0 sits at grid position (0, 0, 0): every rotation angle is 0
    np.testing.assert_allclose(y[:, :, 0, :], ref[:, 0], rtol=1e-13, atol=1e-14)
    # elsewhere each channel pair is only turned, so its length is RMSNorm's
    yp = np.hypot(y[..., 0::2], y[..., 1::2])                     # [B, H, S, D/2]
    rp = np.hypot(ref[..., 0::2], ref[..., 1::2]).transpose(0, 2, 1, 3)
    np.testing.assert_allclose(yp, rp, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("D", [64, 128])
def test_unit_rms_and_scale_invariance(D):
    B, H, grid = 1, 2, (3, 2, 2)
    S = 12
    x = rand_proj(B, S, H, D, 4, scale=3.0)
    y, _ = oracle.norm_rope(x, ones(H * D), grid, eps=0.0)
    per_token = (y**2).sum(axis=(1, 3))  # over heads and channels
    np.testing.assert_allclose(per_token, H * D, rtol=1e-12)
    x4 = gen.f32_to_bf16_bits(gen.bf16_bits_to_f32(x) * 4.0)  # exact in bf16
    y4, _ = oracle.norm_rope(x4, ones(H * D), grid, eps=0.0)
    np.testing.assert_allclose(y4, y, rtol=1e-13, atol=1e-15)


def test_weight_scales_its_channels_only():
    B, S, H, D, grid = 1, 6, 3, 64, (1, 2, 3)
    x = rand_proj(B, S, H, D, 5)
    w = ones(H * D)
    y1, _ = oracle.norm_rope(x, w, grid)
    w2 = w.copy()
    w2[D:2 * D] = 0x4000  # bf16 2.0 on head 1
    y2, _ = oracle.norm_rope(x, w2, grid)
    np.testing.assert_array_equal(y2[:, 0], y1[:, 0])
    np.testing.assert_array_equal(y2[:, 2], y1[:, 2])
    np.testing.assert_allclose(y2[:, 1], 2.0 * y1[:, 1], rtol=1e-15)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("axis", [0, 1, 2])
def test_single_pair_turns_by_the_axis_frequency(D, axis):
    """One nonzero channel pair (a, b) at unit coordinate on one axis: the output pair is
    (a + ib) e^{i phi} / r with phi = theta^(-2i/Da), r the token's RMS; nothing else moves."""
    H, grid, theta, eps = 2, (2, 3, 4), 10000.0, 1e-6
    S = 24
    s = [grid[1] * grid[2], grid[2], 1][axis]  # the token at (1,0,0), (0,1,0) or (0,0,1)
    start, size = segments(D)[axis]
    for i in (0, 1, size // 2 - 1):
        for head in (0, 1):
            a, b = 0.75, -0.5
            x = np.zeros((1, S, H, D), dtype=np.float32)
            c0 = start + 2 * i
            x[0, s, head, c0], x[0, s, head, c0 + 1] = a, b
            y, y16 = oracle.norm_rope(gen.f32_to_bf16_bits(x), ones(H * D), grid, eps=eps, theta=theta)
            r = math.sqrt((a * a + b * b) / (H * D) + eps)
            z = complex(a, b) * cmath.exp(1j * theta ** (-2.0 * i / size)) / r
            got = y[0, head, s]
            assert got[c0] == pytest.approx(z.real, rel=1e-13, abs=1e-15)
            assert got[c0 + 1] == pytest.approx(z.imag, rel=1e-13, abs=1e-15)
            rest = np.delete(y[0, :, s].reshape(-1), [head * D + c0, head * D + c0 + 1])
            assert np.all(rest == 0.0)
            assert y16[0, head, s, c0] == oracle.round_bf16(got[c0])


def test_dot_products_depend_on_position_differences_only():
    """Every token holds the same input: <y_p, y_q> within a head depends on q - p only."""
    H, D, grid = 2, 128, (3, 3, 5)
    S = 45
    row = rand_proj(1, 1, H, D, 6)[0, 0]
    x = np.broadcast_to(row, (1, S, H, D)).copy()
    rng = np.random.default_rng(7)
    w = gen.f32_to_bf16_bits((1.0 + 0.2 * rng.standard_normal(H * D)).astype(np.float32))
    y, _ = oracle.norm_rope(x, w, grid)
    tok = lambda t, hh, ww: (t * grid[1] + hh) * grid[2] + ww
    for h in range(H):
        d1 = y[0, h, tok(0, 0, 0)] @ y[0, h, tok(1, 1, 2)]
        d2 = y[0, h, tok(1, 1, 1)] @ y[0, h, tok(2, 2, 3)]
        d3 = y[0, h, tok(0, 1, 2)] @ y[0, h, tok(1, 2, 4)]
        assert d1 == pytest.approx(d2, rel=1e-12) and d1 == pytest.approx(d3, rel=1e-12)
        self_dots = [y[0, h, s] @ y[0, h, s] for s in range(S)]
        np.testing.assert_allclose(self_dots, self_dots[0], rtol=1e-12)
        # and a different offset gives a different value (the rotation is not trivial)
        d4 = y[0, h, tok(0, 0, 0)] @ y[0, h, tok(1, 1, 3)]
        assert abs(d4 - d1) > 1e-6 * abs(d1)


def test_rounded_output_is_the_nearest_bf16():
    x = rand_proj(1, 12, 2, 64, 8)
    y, y16 = oracle.norm_rope(x, ones(128), (1, 3, 4))
    back = gen.bf16_bits_to_f32(y16).astype(np.float64)
    # |y - back| <= half a bf16 step, i.e. 2^-9 of |y| rounded up to its binade
    step = 2.0 ** (np.floor(np.log2(np.abs(y) + 1e-300)) - 7)
    assert np.all(np.abs(y - back) <= 0.5 * step * (1 + 1e-12))


def test_rejects_bad_grid_and_weight():
    x = rand_proj(1, 12, 2, 64, 9)
    with pytest.raises(ValueError):
        oracle.norm_rope(x, ones(128), (2, 2, 2))
    with pytest.raises(ValueError):
        oracle.norm_rope(x, ones(64), (2, 2, 3))


def test_output_is_rounded_once_from_the_exact_value():
    """All inputs 1 and every weight 1 + 2^-7 put each output at w / sqrt(1 + eps); eps is
    chosen so that this is 1 + 2^-8 + 2^-40, just above a bf16 tie. Rounding the exact value
    gives 1 + 2^-7; a detour through float32 would land on the tie and round down to 1."""
    D = 64
    target = 1.0 + 2.0**-8 + 2.0**-40
    eps = ((1.0 + 2.0**-7) / target) ** 2 - 1.0
    x = np.full((1, 1, 1, D), 0x3F80, dtype=np.uint16)
    w = np.full(D, 0x3F81, dtype=np.uint16)
    y, y16 = oracle.norm_rope(x, w, (1, 1, 1), eps=eps)
    assert np.all(np.abs(y - target) < 2.0**-44)
    assert np.all(y16 == 0x3F81)
