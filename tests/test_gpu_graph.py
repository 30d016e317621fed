"""The calls inside a captured HIP graph: the library allocates nothing, clears nothing with
memset and never synchronises, so a step can be captured once and replayed. Each graph is
replayed several times with eager work and synchronisations in between, and every replay must
reproduce the eager result bit for bit."""
import numpy as np
import pytest
import torch

import dynamic_block_sparse_bsa_amd as bsa
import gen
from parity import to_dev

pytestmark = pytest.mark.gpu


def inputs(D=128, block=128):
    q, k, v = gen.make_qkv(1, 2, 1000, D, 41, grid=(10, 10, 10), alpha=0.5)
    return to_dev(q), to_dev(k), to_dev(v)


def capture(fn):
    """Warm up on a side stream (as torch asks before capture), then capture fn()."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    return g, outs


@pytest.mark.parametrize("D,block", [(128, 128), (64, 64)])
def test_bf16_step_in_a_graph(D, block):
    qd, kd, vd = inputs(D, block)
    r = 0.3

    def step():
        rp, ci = bsa.bsa_select(qd, kd, block, r)
        return rp, ci, bsa.bsa_forward(qd, kd, vd, block, rp, ci)

    ref = [t.clone() for t in step()]
    torch.cuda.synchronize()
    g, outs = capture(step)
    for _ in range(3):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            assert torch.equal(got, want)
        # eager work between replays, on the same inputs
        eager = step()
        torch.cuda.synchronize()
        assert torch.equal(eager[2], ref[2])


def test_fp8_steps_in_a_graph():
    qd, kd, vd = inputs()
    block, r = 128, 0.3

    def fp8_qk():
        rp, ci = bsa.bsa_select(qd, kd, block, r)
        q8, qs = bsa.bsa_quantize_fp8(qd, block)
        k8, ks = bsa.bsa_quantize_fp8(kd, block)
        return (bsa.bsa_forward_fp8(q8, qs, k8, ks, vd, block, rp, ci),)

    def fp8_full():
        rp, ci, q8, qs, k8, ks = bsa.bsa_select_quantize(qd, kd, block, r)
        vt8, vs = bsa.bsa_quantize_v_fp8(vd, block)
        return vt8, vs, bsa.bsa_forward_fp8_full(q8, qs, k8, ks, vt8, vs, block, rp, ci)

    for fn in (fp8_qk, fp8_full):
        ref = [t.clone() for t in fn()]
        torch.cuda.synchronize()
        g, outs = capture(fn)
        for _ in range(3):
            for t in outs:
                t.zero_()
            g.replay()
            torch.cuda.synchronize()
            for got, want in zip(outs, ref):
                assert torch.equal(got, want)
            eager = fn()
            torch.cuda.synchronize()
            assert torch.equal(eager[-1], ref[-1])
    assert np.isfinite(ref[-1].float().cpu().numpy()).all()


@pytest.mark.parametrize("H", [4, 40])
def test_norm_rope_select_in_a_graph(H):
    """The fused RMSNorm + 3D RoPE + selection call and the forward on its outputs, captured
    and replayed (H = 40 takes the kernel's large-LDS launch)."""
    B, D, block, r, grid = 1, 128, 128, 0.3, (4, 8, 12)
    S = 4 * 8 * 12
    xq, xk = gen.make_projections(B, S, H, D, 51, grid=grid, alpha=0.5)
    wq, wk = gen.make_norm_weight(H * D, 52), gen.make_norm_weight(H * D, 53)
    _, _, v = gen.make_qkv(B, H, S, D, 54)
    xqd, xkd, wqd, wkd, vd = to_dev(xq), to_dev(xk), to_dev(wq), to_dev(wk), to_dev(v)

    def step():
        q, k, rp, ci = bsa.bsa_norm_rope_select(xqd, xkd, wqd, wkd, block, grid, r)
        return q, k, rp, ci, bsa.bsa_forward(q, k, vd, block, rp, ci)

    ref = [t.clone() for t in step()]
    torch.cuda.synchronize()
    g, outs = capture(step)
    for _ in range(3):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            assert torch.equal(got, want)
        eager = step()
        torch.cuda.synchronize()
        assert torch.equal(eager[-1], ref[-1])
