"""bsa_select_noalloc, the selection entry point that allocates nothing at call time (its
block means live in the library's per-device scratch array), against bsa_select with a
caller's workspace, through the C ABI. Kept-block lists are integer results: bit-exact."""
import ctypes

import numpy as np
import pytest
import torch

import dynamic_block_sparse_bsa_amd as bsa
import gen
from parity import to_dev

pytestmark = pytest.mark.gpu


def ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def noalloc(q, k, block, r):
    B, H, S, D = q.shape
    n = bsa.bsa_num_blocks(S, block)
    kept = bsa.bsa_num_kept(n, r)
    rows = B * H * n
    rp = torch.full((rows + 1,), -7, dtype=torch.int32, device=q.device)
    ci = torch.full((rows * kept,), -7, dtype=torch.int32, device=q.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    st = bsa._load().bsa_select_noalloc(ptr(q), ptr(k), B, H, S, D, block, r, ptr(rp), ptr(ci), stream)
    assert st == 0, bsa.bsa_last_error()
    return rp, ci


def test_noalloc_select_matches_select_on_two_calls_in_a_row():
    # first call: the 720p workload's shape (B=1, H=40, S=75600, D=128, block 128), seeded noise
    g = torch.Generator(device="cuda").manual_seed(7)
    q = torch.randn(1, 40, 75600, 128, device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn(1, 40, 75600, 128, device="cuda", generator=g).to(torch.bfloat16)
    assert bsa.bsa_select_workspace_bytes(1, 40, 75600, 128, 128) <= bsa.bsa_select_noalloc_max_bytes()
    rp, ci = noalloc(q, k, 128, 0.15)
    ref_rp, ref_ci = bsa.bsa_select(q, k, 128, 0.15)
    torch.cuda.synchronize()
    assert torch.equal(rp, ref_rp) and torch.equal(ci, ref_ci)
    del q, k
    # second call, smaller: D=64, block 64, ragged tail, the locality generator
    qs, ks, _ = gen.make_qkv(2, 3, 2000 - 13, 64, 71, grid=(1987, 1, 1), alpha=0.5)
    qd, kd = to_dev(qs), to_dev(ks)
    rp2, ci2 = noalloc(qd, kd, 64, 0.3)
    ref_rp2, ref_ci2 = bsa.bsa_select(qd, kd, 64, 0.3)
    torch.cuda.synchronize()
    assert torch.equal(rp2, ref_rp2) and torch.equal(ci2, ref_ci2)
    assert int(ci2.min()) >= 0 and rp2.numel() == 2 * 3 * 32 + 1


def test_noalloc_binding_and_repeat():
    qs, ks, _ = gen.make_qkv(1, 2, 1024, 64, 72)
    qd, kd = to_dev(qs), to_dev(ks)
    a = bsa.bsa_select_noalloc(qd, kd, 64, 0.25)
    b = bsa.bsa_select_noalloc(qd, kd, 64, 0.25)
    ref = bsa.bsa_select(qd, kd, 64, 0.25)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, ref)) and all(torch.equal(x, y) for x, y in zip(b, ref))
