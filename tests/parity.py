"""Helpers shared by the GPU parity tests: device transfer and the acceptance criteria.

Criteria (all compare against the CPU oracle in fp64):
  kept-block lists -- bit-exact on every row whose oracle score gap between the k-th and
      (k+1)-th block exceeds 1e-4; on the other rows the GPU list must hold k distinct
      ascending in-range indices and every selected score must be >= every unselected
      score - 1e-4 (oracle scores);
  bf16 attention   -- max abs error <= 2e-2 and mean abs error <= 2e-3;
  fp8-QK attention -- max abs error <= 6e-2 against the unquantised oracle;
  full fp8 attention -- against the exact softmax over the same dequantised Q, K and V
      (oracle.attention_fp8_qkv, no sub-tile schedule): every element within the bound that
      rounding the softmax weights to E4M3 allows, and the mean within the statistical
      bar (see check_fp8_full).
"""
import numpy as np
import torch

import oracle

GAP = 1e-4
BF16_MAX, BF16_MEAN = 2e-2, 2e-3
FP8_MAX = 6e-2
# Full fp8 path. Its operands are the E4M3 codes of Q, K (per-block scales) and V
# (per-channel scales), which the tests compare bit for bit; beyond them it rounds every
# softmax weight to E4M3. Let p_u be the exact weights of a query row (largest 1), w_u the
# stored ones and o = sum p v / sum p the exact result over the dequantised operands. A
# normal E4M3 value is within 2^-4 of what it rounds, a subnormal one within 2^-10 (in
# units of 448 = the largest weight), and a weight formed against an earlier, smaller
# reference point is only scaled down afterwards, so |w_u - p_u| <= eps p_u + eta whatever
# the key order and reference point. Then
#   |sum w v / sum w - o| = |sum (w - p)(v - o)| / sum w
#                         <= (eps sum p|v - o| + eta sum |v - o|) / ((1 - eps) sum p - N eta)
# per channel, with sum p >= 1 and N the row's key count. eps carries 1e-3 for the
# kernel's fp32 logits and rescales; the bf16 output adds at most 2^-8 of |out|.
# Independent roundings of relative size at most 2^-4 give a mean error of order
# 2^-4 sqrt(sum p^2 (v - o)^2); the mean bar is that (with the bf16 output's 2^-9) over all
# elements, which a systematic slip (a stale maximum, a wrong rescale, a wrong scale index)
# exceeds.
FP8_W_EPS = 2.0 ** -4 + 1e-3
FP8_W_ETA = 2.0 ** -10 / 448.0


def to_dev(bits, device="cuda:0"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_lists(gpu_row_ptr, gpu_col, ref):
    """Apply the list criterion; returns (rows bit-exact, rows judged by the tie rule)."""
    kept = ref["kept"]
    s = ref["scores"].reshape(-1, ref["scores"].shape[-1])
    rows, n = s.shape
    rp = np.asarray(gpu_row_ptr)
    assert np.array_equal(rp, np.arange(rows + 1) * kept), "row_ptr is not uniform r*k"
    g = np.asarray(gpu_col).reshape(rows, kept)
    o = ref["col_idx"].reshape(rows, kept)
    clear = ref["gap"] > GAP
    bad = np.nonzero(clear & ~(g == o).all(axis=1))[0]
    assert bad.size == 0, "lists differ on %d clear rows, first %d: gpu %s oracle %s" % (
        bad.size, bad[0], g[bad[0]].tolist(), o[bad[0]].tolist())
    for r in np.nonzero(~clear)[0]:
        row = g[r]
        assert np.all(np.diff(row) > 0) and row[0] >= 0 and row[-1] < n, "row %d malformed: %s" % (r, row)
        sel = np.zeros(n, bool)
        sel[row] = True
        if kept < n:
            assert s[r, sel].min() >= s[r, ~sel].max() - GAP, "row %d violates the tie tolerance" % r
    return int(clear.sum()), int((~clear).sum())


def errors(got, expect):
    e = np.abs(np.asarray(got, dtype=np.float64) - expect)
    return float(e.max()), float(e.mean())


def keys_per_token(row_ptr, col_idx, B, H, S, block, tokens=None):
    """Number of keys each query token attends to (entries outside [0, n) count none)."""
    n = (S + block - 1) // block
    sizes = np.full(n, block, dtype=np.int64)
    sizes[-1] = S - (n - 1) * block
    rp = np.asarray(row_ptr, np.int64)
    ci = np.asarray(col_idx, np.int64)[:rp[-1]]
    ok = (ci >= 0) & (ci < n)
    csum = np.concatenate([[0], np.cumsum(np.where(ok, sizes[np.clip(ci, 0, n - 1)], 0))])
    per_row = csum[rp[1:]] - csum[rp[:-1]]
    t = np.arange(B * H * S) if tokens is None else np.asarray(tokens, np.int64)
    bh, s = np.divmod(t, S)
    keys = per_row[bh * n + s // block]
    return keys if tokens is not None else keys.reshape(B, H, S)


def fp8_full_bound(expect, dev, nkeys):
    """Per-element bound of the full fp8 path around the exact result over its operands."""
    a, b = dev[..., 0, :], dev[..., 1, :]
    denom = (1.0 - FP8_W_EPS) - np.asarray(nkeys, np.float64)[..., None] * FP8_W_ETA
    w = (FP8_W_EPS * a + FP8_W_ETA * b) / denom
    return w + 2.0 ** -8 * (np.abs(expect) + w) + 1e-5


def check_fp8_full(got, expect, dev, nkeys, mean_bar=True):
    """Full fp8 path criteria (see FP8_W_EPS) over outputs whose last axis is D. expect and
    dev come from oracle.attention_fp8_qkv(..., spread=True), nkeys from keys_per_token.
    Returns (max error, mean error, largest error / bound)."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - expect)
    bound = fp8_full_bound(expect, dev, nkeys)
    ratio = float(np.max(err / bound))
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert ratio <= 1.0, ("element beyond the weight-rounding bound", worst, float(err[worst]), float(bound[worst]))
    mx, mean = float(err.max()), float(err.mean())
    if mean_bar:
        bar = float(np.mean(2.0 ** -4 * dev[..., 2, :] + 2.0 ** -9 * np.abs(expect))) + 1e-5
        assert mean <= bar, ("mean error beyond the statistical bar", mean, bar)
    return mx, mean, ratio


def fp8_full_reference(q8, qs, k8, ks, v8, vs, block, row_ptr, col_idx, tokens=None):
    """(expect, dev, nkeys) for check_fp8_full, from the oracle's E4M3 operands (v8 in the
    [B, H, S, D] layout of oracle.quantize_v_fp8)."""
    B, H, S, D = q8.shape
    expect, dev = oracle.attention_fp8_qkv(q8, qs, k8, ks, v8, vs, block, row_ptr, col_idx, tokens=tokens,
                                           spread=True)
    return expect, dev, keys_per_token(row_ptr, col_idx, B, H, S, block, tokens)


def check_fp8_full_vs_unquantised(got, expect, dev, nkeys, exact):
    """The same bound, stated against the unquantised attention: the distance of the exact
    result over the E4M3 operands from it, plus the weight-rounding bound."""
    err = np.abs(np.asarray(got, np.float64) - exact)
    bar = np.abs(expect - exact) + fp8_full_bound(expect, dev, nkeys)
    assert np.all(err <= bar), float(np.max(err - bar))
    return float(err.max()), float(err.mean())
