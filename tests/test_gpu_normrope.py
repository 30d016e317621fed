"""GPU parity of the fused RMSNorm + 3D RoPE + block means (bsa_norm_rope, bsa_norm_rope_select)
against the oracle (oracle.norm_rope: fp64, rounded once to bf16), through the C ABI.

Criteria:
  out   -- the bf16 bits equal the oracle's rounding of the exact value, except where the
           kernel's fp32 arithmetic (a few 2^-24 of the channel pair's length) lands on the
           other side of a rounding midpoint: such elements must be within one bf16 step plus
           that arithmetic error, and at most 1e-3 of all elements may differ;
  means -- |gpu mean - mean of the oracle's bf16 out| <= the block mean of |gpu out - oracle
           out| + 4e-6 * max(1, max |out|): every difference is explained by the elements
           that rounded the other way plus fp32 summation;
  lists -- the list criterion (parity.py) against the oracle's selection run on its own
           bf16 outputs.
"""
import gc

import numpy as np
import pytest
import torch

import dynamic_block_sparse_bsa_amd as bsa
import gen
import oracle
from parity import check_lists, to_dev

pytestmark = pytest.mark.gpu

MAX_DIFF_FRACTION = 1e-3


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def check_out(got16, want16):
    """Returns the fraction of elements whose bf16 bits differ. A differing element may be one
    bf16 step away, plus the absolute error of fp32 arithmetic on its channel pair: a rotated
    value u cos - v sin can cancel to far below |(u, v)|, and there 2^-18 |(u, v)| (sixteen
    times a few fp32 roundings of the pair's length) bounds it."""
    diff = got16 != want16
    frac = float(diff.mean())
    if diff.any():
        idx = np.nonzero(diff.reshape(-1))[0]
        flat = want16.reshape(-1)
        g = gen.bf16_bits_to_f32(got16.reshape(-1)[idx]).astype(np.float64)
        w = gen.bf16_bits_to_f32(flat[idx]).astype(np.float64)
        partner = gen.bf16_bits_to_f32(flat[idx ^ 1]).astype(np.float64)  # the other channel of the pair
        rho = np.hypot(w, partner)
        mag = np.maximum(np.abs(g), np.abs(w))
        step = 2.0 ** (np.floor(np.log2(np.maximum(mag, 2.0**-126))) - 7)
        bad = np.abs(g - w) > step + 2.0**-18 * rho
        assert not bad.any(), "%d elements differ by more than a bf16 step: gpu %r oracle %r" % (
            bad.sum(), g[bad][:4].tolist(), w[bad][:4].tolist())
    assert frac <= MAX_DIFF_FRACTION, "%.2e of the outputs differ" % frac
    return frac


def block_means(a, block):
    """Means over token blocks of a [B, H, S, D] float array (last block partial)."""
    B, H, S, D = a.shape
    n = (S + block - 1) // block
    out = np.empty((B, H, n, D))
    for i in range(n):
        out[:, :, i] = a[:, :, i * block:(i + 1) * block].mean(axis=2)
    return out


def check_means(xbar, got16, want16, block):
    want = oracle.pool(want16, block)
    flips = np.abs(gen.bf16_bits_to_f32(got16).astype(np.float64) - gen.bf16_bits_to_f32(want16))
    bound = block_means(flips, block) + 4e-6 * max(1.0, float(np.abs(want).max()))
    err = np.abs(xbar.cpu().numpy().astype(np.float64) - want)
    assert np.all(err <= bound), "block means differ beyond the rounding flips: max %.3e" % err.max()
    return float(err.max())


# (B, grid, H, D, block): a partial block and a partial 32-token chunk in most; H*D from 64
# (lanes idle) to 5120 (the 14B model's hidden size, > 64 KiB of LDS) and 8192 (the limit).
CASES = [
    (1, (2, 3, 5), 2, 64, 64),
    (2, (3, 10, 10), 3, 128, 128),
    (2, (5, 6, 7), 7, 64, 64),
    (1, (1, 1, 33), 1, 128, 64),
    (1, (3, 5, 37), 40, 128, 128),
    (1, (2, 8, 16), 64, 128, 64),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_S%d_H%d_D%d_b%d" % (c[0], int(np.prod(c[1])), c[2], c[3], c[4]))
def test_norm_rope(case):
    B, grid, H, D, block = case
    S = int(np.prod(grid))
    xq, _ = gen.make_projections(B, S, H, D, 11, grid=grid, alpha=0.5)
    w = gen.make_norm_weight(H * D, 12)
    _, want16 = oracle.norm_rope(xq, w, grid)
    xd = to_dev(xq)
    wd = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    out, xbar = bsa.bsa_norm_rope(xd, wd, block, grid)
    torch.cuda.synchronize()
    got16 = bits(out)
    frac = check_out(got16, want16)
    merr = check_means(xbar, got16, want16, block)
    # the fused means are the means of the written tensor
    pooled = bsa.bsa_pool(out, block)
    np.testing.assert_allclose(xbar.cpu().numpy(), pooled.cpu().numpy(), rtol=0, atol=4e-6 * max(1.0, float(xbar.abs().max())))
    # and without means the same tensor comes out
    out2, none = bsa.bsa_norm_rope(xd, wd, block, grid, means=False)
    torch.cuda.synchronize()
    assert none is None and torch.equal(out2, out)
    print("differing bits %.2e, means max err %.2e" % (frac, merr))


@pytest.mark.parametrize("eps,theta", [(0.0, 10000.0), (1e-2, 500.0)])
def test_norm_rope_eps_and_theta(eps, theta):
    B, grid, H, D, block = 1, (4, 6, 9), 4, 128, 64
    S = int(np.prod(grid))
    xq, _ = gen.make_projections(B, S, H, D, 13, grid=grid, alpha=0.5)
    w = gen.make_norm_weight(H * D, 14)
    _, want16 = oracle.norm_rope(xq, w, grid, eps=eps, theta=theta)
    wd = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    out, xbar = bsa.bsa_norm_rope(to_dev(xq), wd, block, grid, eps=eps, theta=theta)
    torch.cuda.synchronize()
    check_out(bits(out), want16)
    check_means(xbar, bits(out), want16, block)


def run_select_case(B, grid, H, D, block, r, seed):
    S = int(np.prod(grid))
    xq, xk = gen.make_projections(B, S, H, D, seed, grid=grid, alpha=0.5)
    wq, wk = gen.make_norm_weight(H * D, seed + 1), gen.make_norm_weight(H * D, seed + 2)
    _, q16 = oracle.norm_rope(xq, wq, grid, exact=False)
    _, k16 = oracle.norm_rope(xk, wk, grid, exact=False)
    ref = oracle.select(q16, k16, block, r)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    xqd, xkd = to_dev(xq), to_dev(xk)
    del xq, xk
    q, k, rp, ci = bsa.bsa_norm_rope_select(xqd, xkd, dev(wq), dev(wk), block, grid, r)
    torch.cuda.synchronize()
    fq = check_out(bits(q), q16)
    fk = check_out(bits(k), k16)
    exact, ties = check_lists(rp.cpu().numpy(), ci.cpu().numpy(), ref)
    return xqd, xkd, dev(wq), dev(wk), q, k, rp, ci, (fq, fk, exact, ties)


def test_norm_rope_select_small():
    B, grid, H, D, block, r = 2, (4, 12, 20), 4, 128, 64, 0.25
    xqd, xkd, wqd, wkd, q, k, rp, ci, stats = run_select_case(B, grid, H, D, block, r, 21)
    print("differing bits q %.2e k %.2e; lists: %d rows exact, %d near ties" % stats)
    # the same tensors as the single-projection call, and the lists bsa_select finds on them
    q1, _ = bsa.bsa_norm_rope(xqd, wqd, block, grid, means=False)
    k1, _ = bsa.bsa_norm_rope(xkd, wkd, block, grid, means=False)
    rp2, ci2 = bsa.bsa_select(q, k, block, r)
    torch.cuda.synchronize()
    assert torch.equal(q1, q) and torch.equal(k1, k)
    assert torch.equal(rp2, rp)
    same = (ci2 == ci).reshape(-1, bsa.bsa_num_kept(bsa.bsa_num_blocks(int(np.prod(grid)), block), r)).all(dim=1)
    assert float(same.float().mean()) >= 0.99  # fp32 pooling order differs: only near ties may move


@pytest.mark.parametrize("name", ["480p", "720p", "long"])
def test_norm_rope_select_full_size(name):
    """The workloads' shapes (B=1, H=40, D=128, block 128; 480p 21x30x52, 720p 21x45x80,
    long 30x64x64 latent grids with their keep ratios): every output element and every list
    against the oracle."""
    cfg = gen.CONFIGS[name]
    out = run_select_case(cfg["B"], cfg["grid"], cfg["H"], cfg["D"], cfg["block"], cfg["keep_ratio"], 31)
    print("%s: differing bits q %.2e k %.2e; lists: %d rows exact, %d near ties" % ((name,) + out[-1]))
    del out
    gc.collect()
    torch.cuda.empty_cache()
