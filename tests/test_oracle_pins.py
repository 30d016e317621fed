"""Pins for the CPU oracle: each checks it against something other than itself.

Kinds of pin used here: hand-derived cases with closed-form answers (tests/golden), library
routines that the method reduces to in special cases (torch scaled_dot_product_attention
in fp64, numpy means, torch's float8_e4m3fn casts), brute force over all subsets on tiny
inputs, and invariants the definition implies. A plausible slip in the oracle -- a wrong
divisor for a partial block, a dropped 1/sqrt(D), a transposed operand, a flipped tie rule,
zero-padding instead of masking, an off-by-one in k -- fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import gen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16(a):
    return gen.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def f32(b):
    return gen.bf16_bits_to_f32(b)


def as4d(rows, B=1, H=1):
    a = np.asarray(rows, dtype=np.float32)
    return bf16(a.reshape(B, H, a.shape[-2] if a.ndim > 2 else a.shape[0], a.shape[-1]))


def sdpa_f64(q, k, v, mask=None):
    """Library attention (torch, fp64, CPU) on [B,H,S,D] bf16-bit inputs."""
    t = [torch.from_numpy(f32(x).astype(np.float64)) for x in (q, k, v)]
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(t[0], t[1], t[2], attn_mask=m).numpy()


def lists_to_mask(row_ptr, col_idx, B, H, S, block):
    """Boolean [B,H,S,S] mask: query t may see key u iff u's block is in t's block list."""
    n = oracle.num_blocks(S, block)
    mask = np.zeros((B, H, S, S), dtype=bool)
    for bh in range(B * H):
        b, h = divmod(bh, H)
        for i in range(n):
            r = bh * n + i
            for j in col_idx[row_ptr[r]:row_ptr[r + 1]]:
                mask[b, h, i * block:(i + 1) * block, j * block:(j + 1) * block] = True
    return mask


# ---- k rule ----------------------------------------------------------------------------

@pytest.mark.parametrize("n,r,k", [(16, 0.25, 4), (16, 1.0, 16), (256, 0.20, 52), (591, 0.15, 89),
                                   (591, 1.0, 591), (960, 0.10, 96), (3, 0.3, 1), (1, 0.01, 1),
                                   (10, 0.1, 1), (10, 0.11, 2), (7, 0.999, 7)])
def test_num_kept(n, r, k):
    assert oracle.num_kept(n, r) == k


@pytest.mark.parametrize("n,r", [(16, 0.0), (16, -0.1), (16, 1.5), (16, float("nan")), (0, 0.5)])
def test_num_kept_invalid(n, r):
    assert oracle.num_kept(n, r) == 0


def test_num_blocks():
    assert [oracle.num_blocks(S, b) for S, b in [(1024, 64), (75600, 128), (32760, 128), (122880, 128), (1, 128), (129, 128)]] == [16, 591, 256, 960, 1, 2]


# ---- hand cases ------------------------------------------------------------------------

def load_case(name):
    with open(os.path.join(GOLDEN, name)) as f:
        c = json.load(f)
    B, H, S, D = c["B"], c["H"], c["S"], c["D"]
    q, k, v = (bf16(np.array(c[x], dtype=np.float32).reshape(B, H, S, D)) for x in ("q", "k", "v"))
    return c, q, k, v


@pytest.mark.parametrize("name", ["hand_case_a.json", "hand_case_b.json"])
def test_hand_case(name):
    c, q, k, v = load_case(name)
    block, D = c["block"], c["D"]
    np.testing.assert_array_equal(oracle.pool(q, block)[0, 0], np.array(c["expected_qbar"], float))
    np.testing.assert_array_equal(oracle.pool(k, block)[0, 0], np.array(c["expected_kbar"], float))
    sel = oracle.select(q, k, block, c["keep_ratio"])
    assert sel["kept"] == c["expected_kept"]
    np.testing.assert_allclose(sel["scores"][0, 0] * math.sqrt(D), np.array(c["expected_scores_times_sqrtD"], float), rtol=0, atol=1e-14)
    assert sel["col_idx"].tolist() == c["expected_col_idx"]
    if "expected_gap_times_sqrtD" in c:
        np.testing.assert_allclose(sel["gap"] * math.sqrt(D), c["expected_gap_times_sqrtD"], rtol=0, atol=1e-14)
    out = oracle.attention(q, k, v, block, sel["row_ptr"], sel["col_idx"])[0, 0]
    if "expected_out" in c:
        sigma = 1.0 / (1.0 + math.exp(-math.sqrt(2.0)))
        exp = np.array([[a * sigma + b for a, b in row] for row in c["expected_out"]])
        np.testing.assert_allclose(out, exp, rtol=0, atol=1e-14)
    else:
        np.testing.assert_array_equal(out, np.array(c["expected_out_exact"], float))


def test_hand_case_b_zero_padding_would_differ():
    # The golden derivation's counterfactual: a zero key in the partial block would pull
    # tokens 0,1 to (4.4648, -6.2507); the oracle must not.
    c, q, k, v = load_case("hand_case_b.json")
    sel = oracle.select(q, k, c["block"], c["keep_ratio"])
    out = oracle.attention(q, k, v, c["block"], sel["row_ptr"], sel["col_idx"])[0, 0]
    p = 1.0 / (1.0 + math.exp(-3.0 / math.sqrt(2.0)))
    assert abs(out[0, 0] - 5 * p) > 0.5


# ---- library routines in special cases ---------------------------------------------------

def test_dense_equals_library_sdpa_tiny():
    q, k, v, cfg = gen.make_config("tiny")
    sel = oracle.select(q, k, cfg["block"], 1.0)
    assert sel["kept"] == 16
    out = oracle.attention(q, k, v, cfg["block"], sel["row_ptr"], sel["col_idx"])
    ref = sdpa_f64(q, k, v)
    assert np.max(np.abs(out - ref)) <= 1e-12


@pytest.mark.parametrize("S,D,block,r,seed", [(1024, 64, 64, 0.25, 1), (1000, 64, 64, 0.3, 5),
                                              (700, 128, 128, 0.5, 6), (130, 32, 64, 0.5, 7)])
def test_sparse_equals_masked_library_sdpa(S, D, block, r, seed):
    B, H = 2 if S < 1024 else 1, 2
    q, k, v = gen.make_qkv(B, H, S, D, seed)
    sel = oracle.select(q, k, block, r)
    out = oracle.attention(q, k, v, block, sel["row_ptr"], sel["col_idx"])
    mask = lists_to_mask(sel["row_ptr"], sel["col_idx"], B, H, S, block)
    ref = sdpa_f64(q, k, v, mask)
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_pool_equals_numpy_mean_with_ragged_tail():
    B, H, S, D, block = 2, 3, 333, 16, 64
    q, _, _ = gen.make_qkv(B, H, S, D, 11)
    x = f32(q).astype(np.float64)
    got = oracle.pool(q, block)
    n = oracle.num_blocks(S, block)
    for i in range(n):
        np.testing.assert_allclose(got[:, :, i], x[:, :, i * block:(i + 1) * block].mean(axis=2), rtol=1e-13, atol=1e-15)


def test_scores_equal_numpy_product():
    q, k, _, cfg = gen.make_config("tiny")
    qb, kb = oracle.pool(q, cfg["block"]), oracle.pool(k, cfg["block"])
    s = oracle.scores(qb, kb)
    ref = np.matmul(qb, np.swapaxes(kb, -1, -2)) / np.sqrt(cfg["D"])
    np.testing.assert_allclose(s, ref, rtol=1e-13, atol=1e-15)
    # not symmetric in general: a transposed operand would show here
    assert np.max(np.abs(s - np.swapaxes(s, -1, -2))) > 1e-3


def test_topk_brute_force_over_all_subsets():
    """Every 4-subset of 16 blocks: exactly one dominates the rest under (score desc,
    index asc); the oracle must return it. Scores here come from numpy, independently."""
    q, k, _, cfg = gen.make_config("tiny")
    x = lambda t: f32(t).astype(np.float64).reshape(cfg["B"] * cfg["H"], 16, 64, cfg["D"]).mean(axis=2)
    qb, kb = x(q), x(k)
    s = np.einsum("rid,rjd->rij", qb, kb) / np.sqrt(cfg["D"])
    sel = oracle.select(q, k, cfg["block"], cfg["keep_ratio"])
    col = sel["col_idx"].reshape(-1, 4)
    for bh in range(s.shape[0]):
        for i in range(16):
            row = s[bh, i]
            winners = []
            for sub in itertools.combinations(range(16), 4):
                rest = [j for j in range(16) if j not in sub]
                if all((row[a], -a) > (row[b], -b) for a in sub for b in rest):
                    winners.append(sub)
            assert len(winners) == 1
            assert tuple(col[bh * 16 + i]) == winners[0]


def test_gap_equals_library_sorted_difference():
    q, k, _, cfg = gen.make_config("tiny")
    sel = oracle.select(q, k, cfg["block"], cfg["keep_ratio"])
    kk = sel["kept"]
    srt = -np.sort(-sel["scores"].reshape(-1, 16), axis=1)  # descending, numpy's sort
    np.testing.assert_array_equal(sel["gap"], srt[:, kk - 1] - srt[:, kk])
    full = oracle.select(q, k, cfg["block"], 1.0)
    assert np.all(np.isinf(full["gap"]))


# ---- invariants --------------------------------------------------------------------------

def small_int_inputs(B, H, S, D, seed, lo=-4, hi=5):
    rng = np.random.default_rng(seed)
    return tuple(bf16(rng.integers(lo, hi, size=(B, H, S, D)).astype(np.float32)) for _ in range(3))


def test_ones_v_gives_ones_and_constant_v_gives_constant():
    q, k, v, cfg = gen.make_config("tiny")
    sel = oracle.select(q, k, cfg["block"], cfg["keep_ratio"])
    ones = bf16(np.ones(v.shape, np.float32))
    out = oracle.attention(q, k, ones, cfg["block"], sel["row_ptr"], sel["col_idx"])
    assert np.max(np.abs(out - 1.0)) <= 1e-13  # softmax rows sum to 1
    c = np.linspace(-2, 2, cfg["D"], dtype=np.float32)
    const = bf16(np.broadcast_to(c, v.shape).copy())
    out = oracle.attention(q, k, const, cfg["block"], sel["row_ptr"], sel["col_idx"])
    assert np.max(np.abs(out - f32(const[0, 0, 0]))) <= 1e-13


def test_key_shift_invariance():
    B, H, S, D, block = 1, 2, 512, 16, 64
    q, k, v = small_int_inputs(B, H, S, D, 21)
    c = np.random.default_rng(3).integers(-3, 4, size=D).astype(np.float32)
    k2 = bf16(f32(k) + c)  # exact: small integers
    a = oracle.select(q, k, block, 0.25)
    b = oracle.select(q, k2, block, 0.25)
    assert np.all(a["gap"] > 1e-9)
    assert a["col_idx"].tolist() == b["col_idx"].tolist()
    oa = oracle.attention(q, k, v, block, a["row_ptr"], a["col_idx"])
    ob = oracle.attention(q, k2, v, block, b["row_ptr"], b["col_idx"])
    assert np.max(np.abs(oa - ob)) <= 1e-12


def test_query_scale_keeps_lists():
    q, k, _, cfg = gen.make_config("tiny")
    q2 = bf16(f32(q) * 2.0)
    a = oracle.select(q, k, cfg["block"], cfg["keep_ratio"])
    b = oracle.select(q2, k, cfg["block"], cfg["keep_ratio"])
    assert a["col_idx"].tolist() == b["col_idx"].tolist()


def test_permutation_inside_blocks():
    B, H, S, D, block = 1, 2, 640, 32, 64
    q, k, v = gen.make_qkv(B, H, S, D, 9)
    perm = np.concatenate([i * block + np.random.default_rng(i).permutation(block) for i in range(S // block)])
    a = oracle.select(q, k, block, 0.3)
    b = oracle.select(q[:, :, perm], k[:, :, perm], block, 0.3)
    np.testing.assert_allclose(b["scores"], a["scores"], rtol=0, atol=1e-12)
    ok = a["gap"] > 1e-9
    ca, cb = a["col_idx"].reshape(-1, a["kept"]), b["col_idx"].reshape(-1, b["kept"])
    assert np.array_equal(ca[ok], cb[ok])
    oa = oracle.attention(q, k, v, block, a["row_ptr"], a["col_idx"])
    ob = oracle.attention(q[:, :, perm], k[:, :, perm], v[:, :, perm], block, a["row_ptr"], a["col_idx"])
    assert np.max(np.abs(oa[:, :, perm] - ob)) <= 1e-12


def test_duplicate_key_blocks_tie_to_lower_index():
    B, H, S, D, block = 1, 1, 8 * 16, 8, 16
    rng = np.random.default_rng(4)
    q = bf16(np.abs(rng.integers(1, 3, size=(B, H, S, D))).astype(np.float32))  # positive queries
    kf = rng.integers(-1, 2, size=(B, H, S, D)).astype(np.float32)
    kf[:, :, 2 * block:3 * block] = 4.0  # block 2 dominates every row...
    kf[:, :, 5 * block:6 * block] = 4.0  # ...and block 5 is an exact copy of it
    k = bf16(kf)
    sel = oracle.select(q, k, block, 1.0 / 8)
    assert sel["kept"] == 1
    assert sel["col_idx"].tolist() == [2] * 8
    assert np.all(sel["gap"] == 0.0)
    sel2 = oracle.select(q, k, block, 2.0 / 8)
    assert sel2["col_idx"].reshape(-1, 2).tolist() == [[2, 5]] * 8


def test_equal_keys_give_block_mean_of_values():
    B, H, S, D, block = 1, 2, 256, 16, 64
    q, _, v = gen.make_qkv(B, H, S, D, 12)
    k = bf16(np.ones((B, H, S, D), np.float32))
    sel = oracle.select(q, k, block, 0.25)  # k = 1 block per row
    out = oracle.attention(q, k, v, block, sel["row_ptr"], sel["col_idx"])
    vf = f32(v).astype(np.float64)
    n = S // block
    for bh in range(B * H):
        b, h = divmod(bh, H)
        for i in range(n):
            j = sel["col_idx"][bh * n + i]
            ref = vf[b, h, j * block:(j + 1) * block].mean(axis=0)
            np.testing.assert_allclose(out[b, h, i * block:(i + 1) * block], np.broadcast_to(ref, (block, D)), rtol=0, atol=1e-13)


def test_empty_list_gives_zero_rows_and_token_sampling_matches_full():
    B, H, S, D, block = 1, 2, 300, 16, 64
    q, k, v = gen.make_qkv(B, H, S, D, 13)
    n = oracle.num_blocks(S, block)
    lens = np.array([0, 2, 1, 5, 3] * (B * H), dtype=np.int32)
    row_ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng(0)
    col = np.concatenate([np.sort(rng.choice(n, size=L, replace=False)) for L in lens]).astype(np.int32)
    full = oracle.attention(q, k, v, block, row_ptr, col)
    assert np.all(full[:, :, 0:block] == 0.0)
    tok = np.array([5, 70, 299, 300 + 130, 599])
    part = oracle.attention(q, k, v, block, row_ptr, col, tokens=tok)
    np.testing.assert_array_equal(part, full.reshape(-1, D)[tok])
    mask = lists_to_mask(row_ptr, col, B, H, S, block)
    ref = sdpa_f64(q, k, v, mask)  # rows with an empty list are NaN in the library
    sl = np.ones(S, bool)
    sl[0:block] = False
    assert np.max(np.abs(full[:, :, sl] - ref[:, :, sl])) <= 1e-12


def test_malformed_csr_rejected():
    q, k, v = gen.make_qkv(1, 1, 128, 16, 1)
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, 64, np.array([0, 2, 3], np.int32), np.array([1, 0, 0], np.int32))
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, 64, np.array([0, 1, 2], np.int32), np.array([0, 2], np.int32))


# ---- FP8 E4M3FN ------------------------------------------------------------------------

def test_e4m3_decode_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(got[~nan], ref[~nan])
    assert oracle.e4m3_value(0x7E) == 448.0 and oracle.e4m3_value(0x01) == 2.0 ** -9


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.normal(0, 50, 4000), rng.normal(0, 0.01, 2000), rng.uniform(-448, 448, 2000)]).astype(np.float32)
    grid = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)  # exact ties (representable in fp32)
    x = np.concatenate([x, mids, -mids, grid.astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(a)) for a in x], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_quantize_fp8_properties():
    B, H, S, D, block = 1, 2, 300, 32, 128
    x, _, _ = gen.make_qkv(B, H, S, D, 14)
    codes, scale = oracle.quantize_fp8(x, block)
    xf = f32(x)
    n = oracle.num_blocks(S, block)
    for bh in range(B * H):
        b, h = divmod(bh, H)
        for i in range(n):
            blk = xf[b, h, i * block:(i + 1) * block]
            c = codes[b, h, i * block:(i + 1) * block]
            amax = np.max(np.abs(blk))
            assert scale[b, h, i] == np.float32(amax) / np.float32(448.0)
            # the absmax element maps to +-448
            idx = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert c[idx] & 0x7F == 0x7E
            # library cast of the fp32 quotient gives the same codes
            ref = torch.from_numpy(blk / scale[b, h, i]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(c, ref)


def test_fp8_exact_inputs_reduce_to_bf16_attention():
    # Entries on the E4M3 grid with every block's absmax = 448 quantise exactly (scale 1),
    # so the fp8 attention must equal the bf16 attention on the same values.
    B, H, S, D, block = 1, 2, 256, 16, 64
    rng = np.random.default_rng(8)
    grid = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    def on_grid():
        a = rng.choice(grid[grid <= 2.0], size=(B, H, S, D)) * rng.choice([-1, 1], size=(B, H, S, D))
        a[:, :, ::block, 0] = 448.0
        return bf16(a.astype(np.float32))
    q, k = on_grid(), on_grid()
    _, _, v = gen.make_qkv(B, H, S, D, 15)
    q8, qs = oracle.quantize_fp8(q, block)
    k8, ks = oracle.quantize_fp8(k, block)
    assert np.all(qs == 1.0) and np.all(ks == 1.0)
    sel = oracle.select(q, k, block, 0.5)
    a = oracle.attention(q, k, v, block, sel["row_ptr"], sel["col_idx"])
    b = oracle.attention_fp8(q8, qs, k8, ks, v, block, sel["row_ptr"], sel["col_idx"])
    assert np.max(np.abs(a - b)) <= 1e-13


def random_e4m3_codes(rng, shape):
    """Uniform over the 254 finite E4M3FN codes (both NaN patterns excluded)."""
    c = rng.integers(0, 254, size=shape).astype(np.uint8)
    return np.where(c >= 0x7F, c + 1, c).astype(np.uint8)  # skip 0x7F; 0xFF is never drawn


def dequant_torch(codes, scale_rows):
    """Library decode of E4M3FN codes (torch's float8_e4m3fn) times a broadcast scale."""
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy() * scale_rows


def block_scales_to_tokens(scale, S, block):
    """[B, H, n] per-block scales -> [B, H, S, 1] per-token scales."""
    return np.repeat(scale.astype(np.float64), block, axis=2)[:, :, :S, None]


def sdpa_f64_values(q, k, v, mask):
    t = [torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)) for x in (q, k, v)]
    return torch.nn.functional.scaled_dot_product_attention(t[0], t[1], t[2], attn_mask=torch.from_numpy(mask)).numpy()


def random_lists(rng, B, H, n, k):
    rows = B * H * n
    col = np.concatenate([np.sort(rng.choice(n, size=k, replace=False)) for _ in range(rows)]).astype(np.int32)
    return (np.arange(rows + 1) * k).astype(np.int32), col


def check_fp8_qk_random_scales():
    """attention_fp8 on random E4M3 codes with random per-block scales (different for Q and
    K, spread over four binades) equals library attention on the values dequantised by
    torch's float8_e4m3fn decode and the scales repeated over each block's tokens."""
    B, H, S, D, block = 1, 3, 200, 16, 64
    rng = np.random.default_rng(91)
    n = oracle.num_blocks(S, block)
    q8 = random_e4m3_codes(rng, (B, H, S, D))
    k8 = random_e4m3_codes(rng, (B, H, S, D))
    qs = np.exp2(rng.uniform(-12, -8, size=(B, H, n))).astype(np.float32)
    ks = np.exp2(rng.uniform(-12, -8, size=(B, H, n))).astype(np.float32)
    _, _, v = gen.make_qkv(B, H, S, D, 92)
    rp, ci = random_lists(rng, B, H, n, 2)
    got = oracle.attention_fp8(q8, qs, k8, ks, v, block, rp, ci)
    qv = dequant_torch(q8, block_scales_to_tokens(qs, S, block))
    kv = dequant_torch(k8, block_scales_to_tokens(ks, S, block))
    want = sdpa_f64_values(qv, kv, f32(v).astype(np.float64), lists_to_mask(rp, ci, B, H, S, block))
    assert np.max(np.abs(got - want)) <= 1e-12


def test_fp8_qk_random_scales_equal_library_attention_on_dequantised_operands():
    check_fp8_qk_random_scales()


def check_fp8_qkv_random_scales():
    """attention_fp8_qkv (the full FP8 path's operands, exact softmax) on random codes with
    random per-block Q/K scales and per-channel V scales equals library attention on the
    torch-decoded values; its spread terms equal a direct evaluation from the library's
    softmax weights."""
    B, H, S, D, block = 1, 2, 190, 16, 64
    rng = np.random.default_rng(93)
    n = oracle.num_blocks(S, block)
    q8, k8, v8 = (random_e4m3_codes(rng, (B, H, S, D)) for _ in range(3))
    qs = np.exp2(rng.uniform(-12, -8, size=(B, H, n))).astype(np.float32)
    ks = np.exp2(rng.uniform(-12, -8, size=(B, H, n))).astype(np.float32)
    vs = np.exp2(rng.uniform(-9, -5, size=(B, H, D))).astype(np.float32)
    rp, ci = random_lists(rng, B, H, n, 2)
    got, dev = oracle.attention_fp8_qkv(q8, qs, k8, ks, v8, vs, block, rp, ci, spread=True)
    qv = dequant_torch(q8, block_scales_to_tokens(qs, S, block))
    kv = dequant_torch(k8, block_scales_to_tokens(ks, S, block))
    vv = dequant_torch(v8, vs.astype(np.float64)[:, :, None, :])
    mask = lists_to_mask(rp, ci, B, H, S, block)
    want = sdpa_f64_values(qv, kv, vv, mask)
    assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.abs(want).max())
    logits = torch.from_numpy(qv) @ torch.from_numpy(kv).transpose(-1, -2) / math.sqrt(D)
    p = torch.softmax(logits.masked_fill(~torch.from_numpy(mask), float("-inf")), dim=-1).numpy()
    e = np.abs(vv[:, :, None, :, :] - want[:, :, :, None, :])       # [B, H, S(query), S(key), D]
    on = mask[..., None]
    a = np.sum(p[..., None] * e, axis=3)
    b = np.sum(np.where(on, e, 0.0), axis=3)
    r = np.sqrt(np.sum((p[..., None] * e) ** 2, axis=3))
    assert np.allclose(dev[..., 0, :], a, rtol=1e-10, atol=1e-14)
    assert np.allclose(dev[..., 1, :], b, rtol=1e-10, atol=1e-14)
    assert np.allclose(dev[..., 2, :], r, rtol=1e-10, atol=1e-14)


def test_fp8_qkv_random_scales_equal_library_attention_on_dequantised_operands():
    check_fp8_qkv_random_scales()


def test_fp8_qkv_with_unit_scales_equals_the_bf16_definition():
    # E4M3 values of magnitude <= 2 are bf16-exact; with every scale 1 the three operands
    # are the same numbers as their bf16 patterns, so the result is oracle.attention's.
    B, H, S, D, block = 1, 2, 256, 16, 64
    rng = np.random.default_rng(94)
    n = oracle.num_blocks(S, block)
    codes = [random_e4m3_codes(rng, (B, H, S, D)) & np.uint8(0xBF) for _ in range(3)]  # exponent <= 7: |x| < 2
    vals = [dequant_torch(c, 1.0) for c in codes]
    bits = [bf16(x.astype(np.float32)) for x in vals]
    assert all(np.array_equal(f32(b_), x) for b_, x in zip(bits, vals))
    sel = oracle.select(bits[0], bits[1], block, 0.5)
    one_n = np.ones((B, H, n), np.float32)
    got = oracle.attention_fp8_qkv(codes[0], one_n, codes[1], one_n, codes[2], np.ones((B, H, D), np.float32), block,
                                   sel["row_ptr"], sel["col_idx"])
    want = oracle.attention(bits[0], bits[1], bits[2], block, sel["row_ptr"], sel["col_idx"])
    assert np.max(np.abs(got - want)) <= 1e-13


# ---- full FP8 path: P and V in E4M3 as well --------------------------------------------

def e4m3_round(x):
    """Library rounding to E4M3FN (torch's cast), back to fp64."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def dequant(codes, scale_bcast):
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * scale_bcast


def full_fp8_inputs(B, H, S, D, block, seed, qzero=False):
    q, k, v = gen.make_qkv(B, H, S, D, seed)
    if qzero:
        q = np.zeros_like(q)
    q8, qs = oracle.quantize_fp8(q, block)
    k8, ks = oracle.quantize_fp8(k, block)
    v8, vs = oracle.quantize_v_fp8(v)
    return q, k, v, q8, qs, k8, ks, v8, vs


def test_quantize_v_fp8_matches_torch_cast():
    B, H, S, D = 1, 2, 300, 32
    _, _, v = gen.make_qkv(B, H, S, D, 40)
    v[0, 1, :, 5] = 0  # an all-zero channel gets scale 1
    codes, scale = oracle.quantize_v_fp8(v)
    vf = f32(v)
    amax = np.max(np.abs(vf), axis=2)  # [B, H, D]
    expect = np.where(amax > 0, amax.astype(np.float32) / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    assert np.array_equal(scale, expect)
    ref = torch.from_numpy((vf / scale[:, :, None, :]).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    assert np.all(codes[0, 1, :, 5] == 0)


def test_fp8_full_constant_v_gives_constant_output():
    # Each channel of V constant: its codes are exactly +-448 and the stored weights,
    # whatever their rounding, normalise to one, so every output row equals V's dequantised
    # row (448 times the fp32 scale; within a few ulp of V itself).
    B, H, S, D, block = 1, 2, 333, 64, 128
    _, _, _, q8, qs, k8, ks, _, _ = full_fp8_inputs(B, H, S, D, block, 41)
    rng = np.random.default_rng(41)
    c = bf16(rng.normal(0, 2, size=(B, H, 1, D)).astype(np.float32))
    v = np.broadcast_to(c, (B, H, S, D)).copy()
    v8, vs = oracle.quantize_v_fp8(v)
    n = oracle.num_blocks(S, block)
    sel = oracle.select(*gen.make_qkv(B, H, S, D, 41)[:2], block, 0.5)
    out = oracle.attention_fp8_full(q8, qs, k8, ks, v8, vs, block, sel["row_ptr"], sel["col_idx"])
    assert np.all(v8 & 0x7F == 0x7E)
    vhat = dequant(v8, vs[:, :, None, :].astype(np.float64))
    assert np.max(np.abs(out - vhat)) <= 1e-12
    assert np.max(np.abs(vhat - f32(c))) <= 1e-6
    assert n == 3


def test_fp8_full_equal_logits_average_v():
    # Q = 0: every logit is 0, every stored weight is exactly 1 (448 is an E4M3 value), so
    # each output row is the plain average of dequantised V over the row's kept keys.
    B, H, S, D, block = 1, 2, 300, 32, 64
    q, k, v, q8, qs, k8, ks, v8, vs = full_fp8_inputs(B, H, S, D, block, 42, qzero=True)
    sel = oracle.select(gen.make_qkv(B, H, S, D, 42)[0], k, block, 0.4)
    out = oracle.attention_fp8_full(q8, qs, k8, ks, v8, vs, block, sel["row_ptr"], sel["col_idx"])
    vhat = dequant(v8, vs[:, :, None, :].astype(np.float64))
    n = oracle.num_blocks(S, block)
    rp, ci = sel["row_ptr"], sel["col_idx"]
    for bh in range(B * H):
        b, h = divmod(bh, H)
        for i in range(n):
            keys = np.concatenate([np.arange(j * block, min(S, (j + 1) * block)) for j in ci[rp[bh * n + i]:rp[bh * n + i + 1]]])
            mean = vhat[b, h, keys].mean(axis=0)
            rows = out[b, h, i * block:min(S, (i + 1) * block)]
            assert np.max(np.abs(rows - mean)) <= 1e-12


def test_fp8_full_reduces_to_direct_formula_when_the_first_sub_tile_holds_the_max():
    # Key u (u < 64) is a large multiple of query u, so for queries 0..63 the row maximum
    # sits in the first 64-key sub-tile of the first kept block: the running maximum never
    # moves afterwards and the method reduces to w_u = E4M3(448 * 2^(x_u - x_max)) / 448,
    # O = sum w v / sum w, computed here with torch's E4M3 cast and decode.
    B, H, S, D, block = 1, 1, 256, 64, 128
    q, k, v = gen.make_qkv(B, H, S, D, 43)
    kf = f32(k)
    kf[0, 0, :64] = 3.0 * f32(q)[0, 0, :64]
    k = bf16(kf)
    q8, qs = oracle.quantize_fp8(q, block)
    k8, ks = oracle.quantize_fp8(k, block)
    v8, vs = oracle.quantize_v_fp8(v)
    n = oracle.num_blocks(S, block)
    rp = np.array([0, 2, 4], np.int32)
    ci = np.array([0, 1, 0, 1], np.int32)
    tokens = np.arange(64)
    out = oracle.attention_fp8_full(q8, qs, k8, ks, v8, vs, block, rp, ci, tokens=tokens)
    qhat = dequant(q8, np.repeat(qs, block, axis=2)[:, :, :S, None].astype(np.float64))[0, 0]
    khat = dequant(k8, np.repeat(ks, block, axis=2)[:, :, :S, None].astype(np.float64))[0, 0]
    vhat = dequant(v8, vs[:, :, None, :].astype(np.float64))[0, 0]
    x = (qhat[:64] @ khat.T) * math.log2(math.e) / math.sqrt(D)  # [64 queries, S keys]
    assert np.all(np.argmax(x, axis=1) == np.arange(64))
    w = e4m3_round(448.0 * np.exp2(x - x.max(axis=1, keepdims=True))) / 448.0
    expect = (w @ vhat) / w.sum(axis=1, keepdims=True)
    assert np.max(np.abs(out - expect)) <= 1e-12
    assert n == 2


def test_fp8_full_within_weight_rounding_bound_of_exact_softmax():
    # Against the exact softmax over the same dequantised Q, K and V, the only difference is
    # the E4M3 rounding of each weight: at most 2^-4 relative for normal values, so the output
    # can move by at most 2 * 2^-4 / (1 - 2^-4) of max |v| (plus a subnormal term that is far
    # smaller here). A dropped or inverted rescale of the earlier sub-tiles, or weights taken
    # against a stale maximum, breaks this by orders of magnitude.
    B, H, S, D, block = 1, 2, 400, 64, 64
    q, k, v, q8, qs, k8, ks, v8, vs = full_fp8_inputs(B, H, S, D, block, 44)
    kf = f32(k)
    for j in range(oracle.num_blocks(S, block)):  # rising logits: the maximum moves often
        kf[:, :, j * block:(j + 1) * block] *= 1.0 + 0.6 * j
    k = bf16(kf)
    k8, ks = oracle.quantize_fp8(k, block)
    sel = oracle.select(q, k, block, 0.5)
    rp, ci = sel["row_ptr"], sel["col_idx"]
    out = oracle.attention_fp8_full(q8, qs, k8, ks, v8, vs, block, rp, ci)
    n = oracle.num_blocks(S, block)
    qhat = dequant(q8, np.repeat(qs, block, axis=2)[:, :, :S, None].astype(np.float64))
    khat = dequant(k8, np.repeat(ks, block, axis=2)[:, :, :S, None].astype(np.float64))
    vhat = dequant(v8, vs[:, :, None, :].astype(np.float64))
    bound = 2 * 2.0 ** -4 / (1 - 2.0 ** -4) * np.max(np.abs(vhat)) + 1e-3
    worst = 0.0
    for bh in range(B * H):
        b, h = divmod(bh, H)
        for i in range(n):
            keys = np.concatenate([np.arange(j * block, min(S, (j + 1) * block)) for j in ci[rp[bh * n + i]:rp[bh * n + i + 1]]])
            qi = qhat[b, h, i * block:min(S, (i + 1) * block)]
            x = qi @ khat[b, h, keys].T / math.sqrt(D)
            p = np.exp(x - x.max(axis=1, keepdims=True))
            exact = (p / p.sum(axis=1, keepdims=True)) @ vhat[b, h, keys]
            worst = max(worst, float(np.max(np.abs(out[b, h, i * block:min(S, (i + 1) * block)] - exact))))
    assert worst <= bound, (worst, bound)
    assert worst > 0.0


def test_fp8_full_sub_tile_is_64_keys():
    # Keys 0..63 identical, keys 64..127 identical and scoring higher: inside each 64-key
    # sub-tile all logits are equal, so every stored weight is exactly 1 (448) when it is
    # formed, and the rescale is exact arithmetic. The result is then the exact softmax of
    # the two logit levels over dequantised V. Sub-tiles of 128 keys would store the first
    # half's weights as an E4M3 rounding of 2^(x_a - x_b) instead.
    B, H, S, D, block = 1, 1, 128, 64, 128
    q, _, v = gen.make_qkv(B, H, S, D, 45)
    qf = f32(q)
    kf = np.empty((B, H, S, D), np.float32)
    kf[0, 0, :64] = 0.05 * qf[0, 0, 0]
    kf[0, 0, 64:] = 0.2 * qf[0, 0, 0]
    k = bf16(kf)
    q8, qs = oracle.quantize_fp8(q, block)
    k8, ks = oracle.quantize_fp8(k, block)
    v8, vs = oracle.quantize_v_fp8(v)
    out = oracle.attention_fp8_full(q8, qs, k8, ks, v8, vs, block, np.array([0, 1], np.int32),
                                    np.array([0], np.int32), tokens=np.array([0]))
    qhat = dequant(q8, qs[0, 0, 0].astype(np.float64))[0, 0, 0]
    khat = dequant(k8, ks[0, 0, 0].astype(np.float64))[0, 0]
    vhat = dequant(v8, vs[:, :, None, :].astype(np.float64))[0, 0]
    x = khat @ qhat / math.sqrt(D)
    xa, xb = x[0], x[64]
    assert np.all(x[:64] == xa) and np.all(x[64:] == xb) and xb > xa + 0.5
    w = np.exp(x - xb)
    expect = (w @ vhat) / w.sum()
    w_rounded = np.concatenate([e4m3_round(448 * np.exp2((xa - xb) * math.log2(math.e)))[None].repeat(64) / 448, np.ones(64)])
    assert np.max(np.abs((w_rounded @ vhat) / w_rounded.sum() - expect)) > 1e-6  # the two readings differ here
    assert np.max(np.abs(out[0] - expect)) <= 1e-12


@pytest.mark.parametrize("seed,rising,S,D,block,r", [(47, False, 1000, 128, 128, 0.3), (48, True, 6 * 128 - 40, 128, 128, 0.6),
                                                   (49, True, 777, 64, 64, 0.5), (50, False, 1090, 64, 128, 0.5)])
def test_fp8_full_schedule_oracle_within_the_schedule_free_bound(seed, rising, S, D, block, r):
    # The 64-key sub-tile oracle (one order of work and one sequence of reference points) is
    # one instance of the full fp8 path: it must meet the schedule-free criterion that the
    # GPU kernel is held to, element bound and mean bar, including rows whose maximum moves.
    from parity import check_fp8_full, keys_per_token
    B, H = 1, 2
    q, k, v = gen.make_qkv(B, H, S, D, seed, grid=(S // 10, 10, 1) if S % 10 == 0 else None, alpha=0.5)
    if rising:
        kf = f32(k)
        for j in range(oracle.num_blocks(S, block)):
            kf[:, :, j * block:(j + 1) * block] *= 1.0 + 0.7 * j
        k = bf16(kf)
    q8, qs = oracle.quantize_fp8(q, block)
    k8, ks = oracle.quantize_fp8(k, block)
    v8, vs = oracle.quantize_v_fp8(v)
    sel = oracle.select(q, k, block, r)
    rp, ci = sel["row_ptr"], sel["col_idx"]
    sched = oracle.attention_fp8_full(q8, qs, k8, ks, v8, vs, block, rp, ci)
    exact, dev = oracle.attention_fp8_qkv(q8, qs, k8, ks, v8, vs, block, rp, ci, spread=True)
    mx, mean, ratio = check_fp8_full(sched, exact, dev, keys_per_token(rp, ci, B, H, S, block))
    assert 0.0 < mx and ratio < 1.0


def test_fp8_qkv_empty_rows_have_zero_output_and_zero_spread():
    # A row with an empty list attends to nothing (reading R13): zero output, and no spread for
    # the full fp8 bound to add, even when the result buffers start out as garbage.
    B, H, S, D, block = 1, 2, 256, 16, 64
    q, k, v = gen.make_qkv(B, H, S, D, 95)
    q8, qs = oracle.quantize_fp8(q, block)
    k8, ks = oracle.quantize_fp8(k, block)
    v8, vs = oracle.quantize_v_fp8(v)
    rp = np.array([0, 0, 2, 2, 4, 4, 4, 5, 5], np.int32)
    ci = np.array([0, 1, 2, 3, 1], np.int32)
    for _ in range(3):
        out, dev = oracle.attention_fp8_qkv(q8, qs, k8, ks, v8, vs, block, rp, ci, spread=True)
        for bh, i in [(0, 0), (0, 2), (1, 1), (1, 3)]:
            rows = slice(i * block, (i + 1) * block)
            assert np.all(out[0, bh, rows] == 0.0) and np.all(dev[0, bh, rows] == 0.0)
        assert np.all(dev[0, 0, block:2 * block, 1] > 0.0)
