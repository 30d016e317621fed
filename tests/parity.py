"""Helpers shared by the GPU parity tests: device transfer and the acceptance criteria.

Criteria (all compare against the CPU oracle in fp64):
  kept-block lists -- bit-exact on every row whose oracle score gap between the k-th and
      (k+1)-th block exceeds 1e-4; on the other rows the GPU list must hold k distinct
      ascending in-range indices and every selected score must be >= every unselected
      score - 1e-4 (oracle scores);
  bf16 attention   -- max abs error <= 2e-2 and mean abs error <= 2e-3;
  fp8-QK attention -- max abs error <= 6e-2 against the unquantised oracle.
"""
import numpy as np
import torch

GAP = 1e-4
BF16_MAX, BF16_MEAN = 2e-2, 2e-3
FP8_MAX = 6e-2


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
