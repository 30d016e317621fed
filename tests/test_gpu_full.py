"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

Every kept-block list is compared with the oracle's (the list criterion in parity.py).
Outputs are compared on sampled query rows, which the oracle computes one by one: a
seeded random sample plus the first and last token of several heads (the last block is
partial at 480p and 720p), on both the oracle's and the GPU's lists.
"""
import functools
import gc

import numpy as np
import pytest
import torch

import dynamic_block_sparse_bsa_amd as bsa
import gen
import oracle
from parity import (BF16_MAX, BF16_MEAN, FP8_MAX, check_fp8_full, check_fp8_full_vs_unquantised, check_lists, errors,
                    fp8_full_reference, to_dev, to_f64)

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=1)
def workload(name):
    q, k, v, cfg = gen.make_config(name)
    ref = oracle.select(q, k, cfg["block"], cfg["keep_ratio"])
    return q, k, v, cfg, ref


def sample_tokens(B, H, S, count=256, seed=0):
    rng = np.random.default_rng(seed)
    edge = []
    for bh in (0, B * H // 2, B * H - 1):
        edge += [bh * S, bh * S + S - 1, bh * S + (S - 1) // 128 * 128]
    return np.unique(np.concatenate([rng.integers(0, B * H * S, count), edge]))


def rows_of(out, tok, D):
    return to_f64(out.reshape(-1, D)[torch.from_numpy(tok).to(out.device)])


@pytest.mark.parametrize("name", ["480p", "720p", "long"])
def test_full_size_bf16(name):
    q, k, v, cfg, ref = workload(name)
    B, H, S, D, block = q.shape + (cfg["block"],)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    rp, ci = bsa.bsa_select(qd, kd, block, cfg["keep_ratio"])
    out = bsa.bsa_forward(qd, kd, vd, block, rp, ci)
    grp, gci = rp.cpu().numpy(), ci.cpu().numpy()
    exact, ties = check_lists(grp, gci, ref)
    print("%s: %d rows bit-exact, %d near-tie rows within tolerance" % (name, exact, ties))

    tok = sample_tokens(B, H, S)
    expect = oracle.attention(q, k, v, block, grp, gci, tokens=tok)
    mx, mean = errors(rows_of(out, tok, D), expect)
    print("%s bf16 on GPU lists: max %.3e mean %.3e over %d rows" % (name, mx, mean, tok.size))
    assert mx <= BF16_MAX and mean <= BF16_MEAN

    orp, oci = torch.from_numpy(ref["row_ptr"]).cuda(), torch.from_numpy(ref["col_idx"]).cuda()
    out2 = bsa.bsa_forward(qd, kd, vd, block, orp, oci)
    expect2 = oracle.attention(q, k, v, block, ref["row_ptr"], ref["col_idx"], tokens=tok)
    mx, mean = errors(rows_of(out2, tok, D), expect2)
    print("%s bf16 on oracle lists: max %.3e mean %.3e" % (name, mx, mean))
    assert mx <= BF16_MAX and mean <= BF16_MEAN
    del qd, kd, vd, out, out2
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,head", [("720p", 0), ("720p", -1), ("long", 0), ("long", -1)],
                         ids=["720p-first-head", "720p-last-head", "long-first-head", "long-last-head"])
def test_full_size_whole_head(name, head):
    """Every output row of one whole head at full size: every query block (the partial last
    one included) and so every workgroup position of the launch, for bf16 on the GPU's and
    the oracle's lists and for fp8-QK against the unquantised attention."""
    q, k, v, cfg, ref = workload(name)
    B, H, S, D, block = q.shape + (cfg["block"],)
    bh = head % (B * H)
    n = oracle.num_blocks(S, block)
    kept = ref["kept"]
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    rp, ci = bsa.bsa_select(qd, kd, block, cfg["keep_ratio"])
    out = bsa.bsa_forward(qd, kd, vd, block, rp, ci)
    orp, oci = torch.from_numpy(ref["row_ptr"]).cuda(), torch.from_numpy(ref["col_idx"]).cuda()
    out_o = bsa.bsa_forward(qd, kd, vd, block, orp, oci)
    q8, qs = bsa.bsa_quantize_fp8(qd, block)
    k8, ks = bsa.bsa_quantize_fp8(kd, block)
    out8 = bsa.bsa_forward_fp8(q8, qs, k8, ks, vd, block, rp, ci)
    torch.cuda.synchronize()
    grp, gci = rp.cpu().numpy(), ci.cpu().numpy()
    tok = bh * S + np.arange(S)
    expect = oracle.attention(q, k, v, block, grp, gci, tokens=tok)

    got = to_f64(out[bh // H, bh % H])
    mx, mean = errors(got, expect)
    print("%s head %d bf16 on GPU lists, all %d rows: max %.3e mean %.3e" % (name, bh, S, mx, mean))
    assert mx <= BF16_MAX and mean <= BF16_MEAN

    # oracle lists: rows whose list differs from the GPU's are recomputed, the rest reuse expect
    g_rows = gci.reshape(-1, kept)[bh * n:(bh + 1) * n]
    o_rows = ref["col_idx"].reshape(-1, kept)[bh * n:(bh + 1) * n]
    differ = np.nonzero(~(g_rows == o_rows).all(axis=1))[0]
    expect_o = expect.copy()
    if differ.size:
        t_d = np.concatenate([np.arange(i * block, min(S, (i + 1) * block)) for i in differ])
        expect_o[t_d] = oracle.attention(q, k, v, block, ref["row_ptr"], ref["col_idx"], tokens=bh * S + t_d)
    mx, mean = errors(to_f64(out_o[bh // H, bh % H]), expect_o)
    print("%s head %d bf16 on oracle lists (%d rows differ): max %.3e mean %.3e" % (name, bh, differ.size, mx, mean))
    assert mx <= BF16_MAX and mean <= BF16_MEAN

    got8 = to_f64(out8[bh // H, bh % H])
    mx, mean = errors(got8, expect)
    print("%s head %d fp8-QK vs unquantised: max %.3e mean %.3e" % (name, bh, mx, mean))
    if name == "720p":  # the fp8 workload's shape: the stated fp8 bar against the true result
        assert mx <= FP8_MAX
    else:
        # the long shape's stronger locality term makes attention peakier, and rounding Q and K
        # to E4M3 alone moves some outputs well past 6e-2 (0.15-0.20 at most over a whole head,
        # mean 4.4e-3); there the kernel is held to the bf16 bar against the oracle on the same
        # E4M3 operands, as on the small shapes
        oq8, oqs = oracle.quantize_fp8(q, block)
        ok8, oks = oracle.quantize_fp8(k, block)
        assert np.array_equal(qs.cpu().numpy(), oqs) and np.array_equal(ks.cpu().numpy(), oks)
        expect8 = oracle.attention_fp8(oq8, oqs, ok8, oks, v, block, grp, gci, tokens=tok)
        mx8, mean8 = errors(got8, expect8)
        print("%s head %d fp8-QK vs the oracle on the same E4M3 operands: max %.3e mean %.3e" % (name, bh, mx8, mean8))
        assert mx8 <= BF16_MAX and mean8 <= BF16_MEAN
    del qd, kd, vd, out, out_o, out8, q8, k8
    gc.collect()
    torch.cuda.empty_cache()


def test_full_size_fp8():
    q, k, v, cfg, ref = workload("fp8")
    B, H, S, D, block = q.shape + (cfg["block"],)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    q8, qs = bsa.bsa_quantize_fp8(qd, block)
    k8, ks = bsa.bsa_quantize_fp8(kd, block)
    oq8, oqs = oracle.quantize_fp8(q, block)
    ok8, oks = oracle.quantize_fp8(k, block)
    assert np.array_equal(qs.cpu().numpy(), oqs) and np.array_equal(ks.cpu().numpy(), oks)
    assert np.array_equal(q8.cpu().numpy(), oq8) and np.array_equal(k8.cpu().numpy(), ok8)
    rp, ci = bsa.bsa_select(qd, kd, block, cfg["keep_ratio"])
    check_lists(rp.cpu().numpy(), ci.cpu().numpy(), ref)
    out = bsa.bsa_forward_fp8(q8, qs, k8, ks, vd, block, rp, ci)
    tok = sample_tokens(B, H, S, seed=1)
    got = rows_of(out, tok, D)
    grp, gci = rp.cpu().numpy(), ci.cpu().numpy()
    expect = oracle.attention(q, k, v, block, grp, gci, tokens=tok)
    mx, mean = errors(got, expect)
    print("fp8 vs unquantised oracle: max %.3e mean %.3e" % (mx, mean))
    assert mx <= FP8_MAX
    expect8 = oracle.attention_fp8(oq8, oqs, ok8, oks, v, block, grp, gci, tokens=tok)
    mx8, mean8 = errors(got, expect8)
    print("fp8 vs oracle on the same E4M3 operands: max %.3e mean %.3e" % (mx8, mean8))
    assert mx8 <= BF16_MAX and mean8 <= BF16_MEAN


def natural_from_vt(vt, B, H, S, D, block):
    """Undo bsa_quantize_v_fp8's transposed, key-permuted layout (defined in include/bsa.h)."""
    n = oracle.num_blocks(S, block)
    S_pad = n * block
    pos = np.arange(64)
    g, e = pos // 32, pos % 32
    key = 32 * (e // 16) + 8 * ((e % 16) // 4) + 4 * g + (e % 16) % 4
    order = np.empty(S_pad, np.int64)
    for grp in range(S_pad // 64):
        order[64 * grp + key] = 64 * grp + pos
    nat = np.asarray(vt).reshape(B * H, D, S_pad)[:, :, order]
    return nat[:, :, :S].transpose(0, 2, 1).reshape(B, H, S, D), nat[:, :, S:]


def test_full_size_fp8_full():
    """The full fp8 path (E4M3 Q, K, V and weights) at the 720p fp8 workload."""
    q, k, v, cfg, ref = workload("fp8")
    B, H, S, D, block = q.shape + (cfg["block"],)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    rp, ci, q8, qs, k8, ks = bsa.bsa_select_quantize(qd, kd, block, cfg["keep_ratio"])
    check_lists(rp.cpu().numpy(), ci.cpu().numpy(), ref)
    oq8, oqs = oracle.quantize_fp8(q, block)
    ok8, oks = oracle.quantize_fp8(k, block)
    assert np.array_equal(qs.cpu().numpy(), oqs) and np.array_equal(ks.cpu().numpy(), oks)
    assert np.array_equal(q8.cpu().numpy(), oq8) and np.array_equal(k8.cpu().numpy(), ok8)
    del oq8, ok8
    vt, vs = bsa.bsa_quantize_v_fp8(vd, block)
    ov8, ovs = oracle.quantize_v_fp8(v)
    codes, pad = natural_from_vt(vt.cpu().numpy(), B, H, S, D, block)
    assert np.array_equal(codes, ov8) and np.all(pad == 0)
    assert np.array_equal(vs.cpu().numpy(), ovs)
    del codes, pad
    gc.collect()
    out = bsa.bsa_forward_fp8_full(q8, qs, k8, ks, vt, vs, block, rp, ci)
    tok = sample_tokens(B, H, S, seed=2)
    got = rows_of(out, tok, D)
    grp, gci = rp.cpu().numpy(), ci.cpu().numpy()
    oq8, oqs = oracle.quantize_fp8(q, block)
    ok8, oks = oracle.quantize_fp8(k, block)
    expect, dev, nkeys = fp8_full_reference(oq8, oqs, ok8, oks, ov8, ovs, block, grp, gci, tokens=tok)
    mx, mean, ratio = check_fp8_full(got, expect, dev, nkeys)
    print("fp8 full vs exact attention on its E4M3 operands: max %.3e mean %.3e, %.2f of the bound" % (mx, mean, ratio))
    exact = oracle.attention(q, k, v, block, grp, gci, tokens=tok)
    mx2, mean2 = check_fp8_full_vs_unquantised(got, expect, dev, nkeys, exact)
    print("fp8 full vs unquantised attention: max %.3e mean %.3e" % (mx2, mean2))
    assert mx2 <= FP8_MAX
    sched = oracle.attention_fp8_full(oq8, oqs, ok8, oks, ov8, ovs, block, grp, gci, tokens=tok)
    print("diagnostic: fp8 full vs the 64-key sub-tile oracle: max %.3e mean %.3e" % errors(got, sched))

    # every row of the last head: every query block (the partial last one included) and so
    # every workgroup position of the launch
    bh = B * H - 1
    tok = bh * S + np.arange(S)
    got = to_f64(out[bh // H, bh % H])
    expect, dev, nkeys = fp8_full_reference(oq8, oqs, ok8, oks, ov8, ovs, block, grp, gci, tokens=tok)
    mx, mean, ratio = check_fp8_full(got, expect, dev, nkeys)
    print("head %d, all %d rows: fp8 full vs exact attention on its E4M3 operands: max %.3e mean %.3e, %.2f of the "
          "bound" % (bh, S, mx, mean, ratio))
    exact = oracle.attention(q, k, v, block, grp, gci, tokens=tok)
    mx2, mean2 = check_fp8_full_vs_unquantised(got, expect, dev, nkeys, exact)
    print("head %d, all rows: fp8 full vs unquantised attention: max %.3e mean %.3e" % (bh, mx2, mean2))
    assert mx2 <= FP8_MAX
