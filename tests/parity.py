"""Helpers shared by the GPU parity tests: device transfer and the acceptance criteria.

Criteria (all compare against the CPU oracle in fp64):
  kept-block lists -- bit-exact on every row whose oracle score gap between the k-th and
      (k+1)-th block exceeds 1e-4; on the other rows the GPU list must hold k distinct
      ascending in-range indices and every selected score must be >= every unselected
      score - 1e-4 (oracle scores);
  bf16 attention   -- max abs error <= 2e-2 and mean abs error <= 2e-3;
  fp8-QK attention -- max abs error <= 6e-2 against the unquantised oracle;
  full fp8 attention -- against the oracle's full-fp8 attention: mean <= 2e-3, max <= 6e-2,
      and at most 1 % of the query rows beyond 2e-2 (see check_fp8_full).
"""
import numpy as np
import torch

GAP = 1e-4
BF16_MAX, BF16_MEAN = 2e-2, 2e-3
FP8_MAX = 6e-2
# Full fp8 path against the oracle that rounds its weights the same way. The two sides
# differ only in fp32 vs fp64 arithmetic, but a weight whose 448 * p lies within that
# difference of an E4M3 midpoint can round one code apart (a relative step of at most 2^-3);
# the flip moves that query's output by at most 2^-3 * (the key's share of the row weight)
# * 2 max|v| -- on every element of that query's row. The bulk must still agree to the bf16
# bar: at most FP8_FULL_OUTLIER_ROWS of the query rows may exceed BF16_MAX anywhere, no
# element FP8_FULL_MAX, and the mean stays at BF16_MEAN.
FP8_FULL_MAX = 6e-2
FP8_FULL_OUTLIER_ROWS = 1e-2


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


def check_fp8_full(got, expect):
    """Full fp8 path criteria (see FP8_FULL_MAX) over outputs whose last axis is D; returns
    (max, mean, fraction of query rows beyond the bf16 bar)."""
    err = np.abs(np.asarray(got, np.float64) - np.asarray(expect, np.float64))
    mx, mean = float(err.max()), float(err.mean())
    frac = float(np.mean(err.max(axis=-1) > BF16_MAX))
    assert mx <= FP8_FULL_MAX and mean <= BF16_MEAN and frac <= FP8_FULL_OUTLIER_ROWS, (mx, mean, frac)
    return mx, mean, frac
