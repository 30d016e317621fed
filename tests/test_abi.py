"""The C-ABI library on the host: it loads, exports every symbol include/bsa.h declares,
implements the k rule like the oracle, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import dynamic_block_sparse_bsa_amd as bsa
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ["bsa_select", "bsa_forward", "bsa_quantize_fp8", "bsa_forward_fp8", "bsa_pool",
                 "bsa_num_blocks", "bsa_num_kept", "bsa_select_workspace_bytes", "bsa_check_csr",
                 "bsa_status_string", "bsa_last_error"]:
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(bsa.lib_path)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert missing == []


def test_k_rule_matches_oracle():
    rng = np.random.default_rng(0)
    cases = [(n, r) for n in [1, 2, 3, 16, 255, 256, 591, 960, 8192] for r in [0.01, 0.1, 0.15, 0.2, 0.25, 0.3, 0.5, 1.0]]
    cases += [(int(n), float(r)) for n, r in zip(rng.integers(1, 5000, 300), rng.uniform(0, 1, 300))]
    cases += [(16, 0.0), (16, -1.0), (16, 1.0000001), (16, float("nan")), (0, 0.5), (-3, 0.5)]
    for n, r in cases:
        assert bsa.bsa_num_kept(n, r) == oracle.num_kept(n, r), (n, r)
    for S, b in [(1, 64), (64, 64), (65, 64), (75600, 128), (0, 64), (5, 0)]:
        assert bsa.bsa_num_blocks(S, b) == oracle.num_blocks(S, b)


def test_workspace_bytes():
    assert bsa.bsa_select_workspace_bytes(1, 40, 75600, 128, 128) == 2 * 40 * 591 * 128 * 4
    assert bsa.bsa_select_workspace_bytes(1, 1, 1, 64, 64) == 512
    assert bsa.bsa_select_workspace_bytes(0, 1, 1, 64, 64) == 0


def test_status_strings():
    for code, name in bsa.STATUS_NAMES.items():
        assert bsa.bsa_status_string(code) == name


def lib():
    return bsa._load()


FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: every case below fails first


@pytest.mark.parametrize("args,status", [
    # B < 1
    (dict(B=0), 1),
    # unsupported head dim and block
    (dict(D=96), 2), (dict(block=32), 2),
    # null q
    (dict(q=None), 1),
    # misaligned k
    (dict(k=ctypes.c_void_p(0x10008)), 1),
    # keep ratio outside (0, 1]
    (dict(r=0.0), 1), (dict(r=1.5), 1), (dict(r=float("nan")), 1),
    # workspace too small
    (dict(ws_bytes=100), 3),
    # too many blocks for selection
    (dict(S=8193 * 64, block=64), 2),
])
def test_select_rejects_bad_arguments(args, status):
    a = dict(q=FAKE, k=FAKE, B=1, H=2, S=1024, D=64, block=64, r=0.25, rp=FAKE, ci=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(args)
    st = lib().bsa_select(a["q"], a["k"], a["B"], a["H"], a["S"], a["D"], a["block"], a["r"], a["rp"], a["ci"],
                          a["ws"], a["ws_bytes"], None)
    assert st == status, bsa.bsa_last_error()
    assert bsa.bsa_last_error() != ""


@pytest.mark.parametrize("args,status", [
    (dict(S=0), 1), (dict(D=32), 2), (dict(v=None), 1), (dict(out=ctypes.c_void_p(0x10004)), 1),
    (dict(rp=ctypes.c_void_p(0x10002)), 1), (dict(out=ctypes.c_void_p(0x10000)), 1),  # out aliases q
])
def test_forward_rejects_bad_arguments(args, status):
    a = dict(q=ctypes.c_void_p(0x10000), k=ctypes.c_void_p(0x20000), v=ctypes.c_void_p(0x30000), B=1, H=2, S=1024,
             D=64, block=64, rp=FAKE, ci=FAKE, out=ctypes.c_void_p(0x40000))
    a.update(args)
    st = lib().bsa_forward(a["q"], a["k"], a["v"], a["B"], a["H"], a["S"], a["D"], a["block"], a["rp"], a["ci"],
                           a["out"], None)
    assert st == status, bsa.bsa_last_error()


def test_fp8_calls_reject_bad_arguments():
    st = lib().bsa_quantize_fp8(FAKE, 1, 1, 128, 128, 128, None, FAKE, None)
    assert st == 1
    st = lib().bsa_forward_fp8(FAKE, None, FAKE, FAKE, FAKE, 1, 1, 128, 128, 128, FAKE, FAKE, ctypes.c_void_p(0x50000), None)
    assert st == 1
    st = lib().bsa_pool(FAKE, 1, 1, 128, 80, 128, FAKE, None)
    assert st == 2


def P(a):
    return ctypes.c_void_p(a)


QA, KA, VA, RPA, CIA = 0x1000000, 0x2000000, 0x3000000, 0x4000000, 0x5000000
TENSOR = 2 * 1024 * 64 * 2  # B=1, H=2, S=1024, D=64, bf16


@pytest.mark.parametrize("out_at", [QA + 16, QA + TENSOR - 16, QA - TENSOR + 4096, VA + 4096, RPA - TENSOR + 64],
                         ids=["q-start", "q-end", "ends-in-q", "in-v", "over-row_ptr"])
def test_forward_rejects_any_overlap_of_out(out_at):
    """out overlapping any part of q, v or row_ptr is refused, not only out == q."""
    st = lib().bsa_forward(P(QA), P(KA), P(VA), 1, 2, 1024, 64, 64, P(RPA), P(CIA), P(out_at), None)
    assert st == 1 and "overlap" in bsa.bsa_last_error(), bsa.bsa_last_error()


def test_fp8_forwards_reject_out_over_their_operands():
    # fp8 operands are 1 byte per element, the transposed full-fp8 V holds bsa_vt_fp8_bytes
    st = lib().bsa_forward_fp8(P(QA), P(0x6000000), P(KA), P(0x7000000), P(VA), 1, 2, 1024, 64, 64, P(RPA), P(CIA),
                               P(KA + TENSOR // 2 - 32), None)
    assert st == 1 and "overlap" in bsa.bsa_last_error()
    vt = bsa.bsa_vt_fp8_bytes(1, 2, 1024, 64, 64)
    st = lib().bsa_forward_fp8_full(P(QA), P(0x6000000), P(KA), P(0x7000000), P(VA), P(0x8000000), 1, 2, 1024, 64, 64,
                                    P(RPA), P(CIA), P(VA + vt - 32), None)
    assert st == 1 and "overlap" in bsa.bsa_last_error()


def test_select_and_quantisers_reject_overlapping_outputs():
    big = 1 << 30
    # col_idx (2*16*4 entries) running into the workspace
    st = lib().bsa_select(P(0x10000), P(0x100000), 1, 2, 1024, 64, 64, 0.25, P(0x200000), P(0x300000),
                          P(0x300000 + 64), big, None)
    assert st == 1 and "overlap" in bsa.bsa_last_error()
    # row_ptr inside k
    st = lib().bsa_select(P(0x10000), P(0x100000), 1, 2, 1024, 64, 64, 0.25, P(0x100000 + 4096), P(0x300000),
                          P(0x400000), big, None)
    assert st == 1
    # codes over the input
    st = lib().bsa_quantize_fp8(P(0x10000), 1, 2, 1024, 64, 64, P(0x10000 + 1024), P(0x200000), None)
    assert st == 1
    st = lib().bsa_quantize_v_fp8(P(0x10000), 1, 2, 1024, 64, 64, P(0x200000), P(0x200000 + 4096), None)
    assert st == 1
    st = lib().bsa_pool(P(0x10000), 1, 2, 1024, 64, 64, P(0x10000 + 64 * 1024), None)
    assert st == 1


def test_binding_checks_caller_buffers_before_any_launch(monkeypatch):
    """Undersized or misshapen outputs, CSR arrays of the wrong length and short workspaces
    raise ValueError (TypeError for a wrong dtype) in the binding, before the library is asked
    to launch anything. (The device check is relaxed to CPU tensors here; nothing reaches a
    HIP call.)"""
    import torch

    real = bsa._dev_tensor

    def cpu_ok(t, name, dtypes, ndim=4):
        if isinstance(t, torch.Tensor) and t.device.type == "cpu":
            if t.dtype not in dtypes:
                raise TypeError(name)
            if ndim is not None and t.dim() != ndim:
                raise ValueError(name)
            if not t.is_contiguous():
                raise ValueError(name)
            return t
        return real(t, name, dtypes, ndim)

    monkeypatch.setattr(bsa, "_dev_tensor", cpu_ok)
    monkeypatch.setattr(bsa, "_stream", lambda t: (_ for _ in ()).throw(AssertionError("reached a launch")))
    B, H, S, D, block = 1, 2, 300, 64, 64
    n = bsa.bsa_num_blocks(S, block)
    rows = B * H * n
    q = torch.zeros(B, H, S, D, dtype=torch.bfloat16)
    rp = torch.zeros(rows + 1, dtype=torch.int32)
    ci = torch.zeros(rows * 2, dtype=torch.int32)
    bad = [
        lambda: bsa.bsa_forward(q, q, q, block, rp, ci, out=torch.empty(B, H, S - 1, D, dtype=torch.bfloat16)),
        lambda: bsa.bsa_forward(q, q, q, block, rp[:-1], ci),
        lambda: bsa.bsa_forward(q, q, q, block, rp, ci, out=torch.empty(B, H, S, D, dtype=torch.float32)),
        lambda: bsa.bsa_pool(q, block, out=torch.empty(B, H, n - 1, D, dtype=torch.float32)),
        lambda: bsa.bsa_select(q, q, block, 0.5, row_ptr=torch.empty(rows, dtype=torch.int32)),
        lambda: bsa.bsa_select(q, q, block, 0.5, col_idx=torch.empty(rows * 2 - 1, dtype=torch.int32)),
        lambda: bsa.bsa_select(q, q, block, 0.5, workspace=torch.empty(16, dtype=torch.uint8)),
        lambda: bsa.bsa_quantize_fp8(q, block, codes=torch.empty(B, H, S, D - 1, dtype=torch.uint8)),
        lambda: bsa.bsa_quantize_fp8(q, block, scale=torch.empty(rows - 1, dtype=torch.float32)),
        lambda: bsa.bsa_quantize_v_fp8(q, block, scale=torch.empty(B * H * D - 1, dtype=torch.float32)),
        lambda: bsa.bsa_select_quantize(q, q, block, 0.5, col_idx=torch.empty(1, dtype=torch.int32)),
    ]
    for i, f in enumerate(bad):
        with pytest.raises((ValueError, TypeError)):
            f()
    x = torch.zeros(B, S, H, D, dtype=torch.bfloat16)
    w = torch.zeros(H * D, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        bsa.bsa_norm_rope(x, w, block, (3, 10, 10), out=torch.empty(B, H, S, D - 8, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        bsa.bsa_norm_rope(x, w, block, (3, 10, 10), xbar=torch.empty(1, dtype=torch.float32))


def test_noalloc_select_rejects_shapes_beyond_its_scratch():
    # 2*B*H*n*D*4 bytes of means: 80 heads of 960 blocks at D=128 need 78.6 MB > 64 MiB
    assert bsa.bsa_select_noalloc_max_bytes() == 64 << 20
    st = lib().bsa_select_noalloc(P(0x1000000), P(0x40000000), 1, 80, 122880, 128, 128, 0.1, P(0x80000000),
                                  P(0x90000000), None)
    assert st == 2 and "at most" in bsa.bsa_last_error(), bsa.bsa_last_error()
    st = lib().bsa_select_noalloc(None, P(0x40000000), 1, 2, 1024, 64, 64, 0.25, P(0x80000000), P(0x90000000), None)
    assert st == 1


def gpu_visible():
    import torch
    return torch.cuda.is_available()


def test_no_device_status_without_gpu():
    if gpu_visible():
        pytest.skip("a GPU is visible; this checks the no-device path")
    a = [ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000)]
    st = lib().bsa_forward(a[0], a[1], a[2], 1, 1, 128, 128, 128, ctypes.c_void_p(0x50000), FAKE,
                           ctypes.c_void_p(0x40000), None)
    assert st == 4, bsa.bsa_last_error()
    st = lib().bsa_select(a[0], a[1], 1, 1, 128, 128, 128, 0.5, ctypes.c_void_p(0x50000), ctypes.c_void_p(0x60000),
                          ctypes.c_void_p(0x70000), 1 << 20, None)
    assert st == 4, bsa.bsa_last_error()


def test_check_csr():
    bsa.bsa_check_csr(np.array([0, 2, 3]), np.array([0, 3, 1]), 2, 4)
    bsa.bsa_check_csr(np.array([0, 2, 3]), np.array([0, 3, 1, 99]), 2, 4)  # spare entries are not read
    for rp, ci in [([0, 2, 3], [1, 0, 0]), ([0, 2, 3], [0, 4, 1]), ([1, 2, 3], [0, 1, 2]), ([0, 2, 1], [0, 1]),
                   ([0, 1, 2], [0, -1]),
                   ([0, 2, 3], [0, 3]),  # row 1 ends past col_idx (checked in C, from the length passed)
                   ([0, 2], [0, 1]), ([0, 1, 2, 3], [0, 1, 2])]:  # row_ptr not rows + 1 long
        with pytest.raises(bsa.BsaError) as e:
            bsa.bsa_check_csr(np.array(rp), np.array(ci), 2, 4)
        assert e.value.status == 1


def test_binding_requires_device_tensors():
    import torch
    x = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        bsa.bsa_forward(x, x, x, 64, torch.zeros(2, dtype=torch.int32), torch.zeros(1, dtype=torch.int32))


def test_full_fp8_calls_check_arguments_on_the_host():
    A = ctypes.c_void_p
    # bytes of the transposed V codes: B*H*D*ceil(S/block)*block
    assert bsa.bsa_vt_fp8_bytes(1, 40, 75600, 128, 128) == 40 * 128 * 591 * 128
    assert bsa.bsa_vt_fp8_bytes(2, 3, 1, 64, 64) == 2 * 3 * 64 * 64
    assert bsa.bsa_vt_fp8_bytes(0, 1, 1, 64, 64) == 0
    # null v_scale / misaligned v_scale for the full fp8 forward
    st = lib().bsa_forward_fp8_full(FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 128, 128, 128, FAKE, FAKE, A(0x50000), None)
    assert st == 1, bsa.bsa_last_error()
    st = lib().bsa_forward_fp8_full(FAKE, FAKE, FAKE, FAKE, FAKE, A(0x60004), 1, 1, 128, 128, 128, FAKE, FAKE, A(0x50000), None)
    assert st == 1
    # unsupported shapes and a one-(b, h) slice too long for 32-bit buffer offsets
    st = lib().bsa_quantize_v_fp8(FAKE, 1, 1, 128, 96, 128, FAKE, FAKE, None)
    assert st == 2
    st = lib().bsa_quantize_v_fp8(FAKE, 1, 1, 1 << 23, 128, 128, FAKE, FAKE, None)
    assert st == 2, bsa.bsa_last_error()
    # select_quantize: keep_ratio and workspace checked before any device work
    st = lib().bsa_select_quantize(FAKE, FAKE, 1, 1, 1024, 64, 64, 0.0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   1 << 20, None)
    assert st == 1
    st = lib().bsa_select_quantize(FAKE, FAKE, 1, 1, 1024, 64, 64, 0.5, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None)
    assert st == 3


C_CONSUMER = r"""
#include <stdio.h>
#include "bsa.h"
int main(void) {
    int32_t n = bsa_num_blocks(1000, 128);
    int32_t k = bsa_num_kept(n, 0.3);
    bsa_status st = bsa_select(NULL, NULL, 1, 1, 1000, 128, 128, 0.3, NULL, NULL, NULL, 0, NULL);
    printf("%d %d %d %s\n", (int)n, (int)k, (int)st, bsa_status_string(st));
    return 0;
}
"""


def test_header_is_plain_c_and_links(tmp_path):
    """include/bsa.h compiles as strict C99 and a C program links against libbsa.so."""
    import shutil
    import subprocess

    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = tmp_path / "consumer.c"
    src.write_text(C_CONSUMER)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(bsa.lib_path)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
           "-L", libdir, "-lbsa", "-Wl,-rpath," + libdir, "-Wl,-rpath-link,/opt/rocm/lib", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    n, k, st, name = out.stdout.split()
    assert (int(n), int(k)) == (8, bsa.bsa_num_kept(8, 0.3))
    assert name == "BSA_ERR_INVALID_ARGUMENT" and int(st) != 0


def test_norm_rope_workspace_bytes():
    # partial sums of 32-token chunks: B * ceil(S/32) * H*D floats, rounded up to 256
    assert bsa.bsa_norm_rope_workspace_bytes(1, 40, 75600, 128) == 2363 * 5120 * 4
    assert bsa.bsa_norm_rope_workspace_bytes(2, 1, 33, 64) == 2 * 2 * 64 * 4  # two chunks per sequence
    assert bsa.bsa_norm_rope_workspace_bytes(1, 1, 1, 64) == 256
    assert bsa.bsa_norm_rope_workspace_bytes(0, 1, 1, 64) == 0
    sel = bsa.bsa_select_workspace_bytes(1, 40, 75600, 128, 128)
    assert bsa.bsa_norm_rope_select_workspace_bytes(1, 40, 75600, 128, 128) == 2 * 2363 * 5120 * 4 + sel


@pytest.mark.parametrize("args,status", [
    (dict(B=0), 1), (dict(D=96), 2), (dict(block=32), 2),
    (dict(H=65), 2),                                    # H*D = 8320 > 8192
    (dict(x=None), 1), (dict(w=ctypes.c_void_p(0x20008)), 1), (dict(out=None), 1),
    (dict(gt=2), 1), (dict(gh=0), 1),                   # grid does not hold S tokens
    (dict(eps=-1e-6), 1), (dict(eps=float("inf")), 1), (dict(theta=0.0), 1), (dict(theta=float("nan")), 1),
    (dict(out=ctypes.c_void_p(0x10000 + 4096)), 1),     # out overlaps x
    (dict(ws=None), 1), (dict(ws_bytes=16), 3), (dict(xbar=ctypes.c_void_p(0x60002)), 1),
])
def test_norm_rope_rejects_bad_arguments(args, status):
    a = dict(x=ctypes.c_void_p(0x10000), w=ctypes.c_void_p(0x20000), B=1, H=4, S=12, D=128, block=64, gt=1, gh=3,
             gw=4, eps=1e-6, theta=1e4, out=ctypes.c_void_p(0x1000000), xbar=ctypes.c_void_p(0x60000), ws=FAKE,
             ws_bytes=1 << 30)
    a.update(args)
    st = lib().bsa_norm_rope(a["x"], a["w"], a["B"], a["H"], a["S"], a["D"], a["block"], a["gt"], a["gh"], a["gw"],
                             a["eps"], a["theta"], a["out"], a["xbar"], a["ws"], a["ws_bytes"], None)
    assert st == status, bsa.bsa_last_error()


@pytest.mark.parametrize("args,status", [
    (dict(r=0.0), 1), (dict(r=1.5), 1), (dict(rp=None), 1), (dict(ws_bytes=1024), 3),
    (dict(k_out=ctypes.c_void_p(0x1000000 + 64)), 1),    # q_out and k_out overlap
    (dict(k_out=ctypes.c_void_p(0x10000)), 1),           # k_out overlaps xq
    (dict(gw=5), 1),
    # too many blocks for selection (tensors far apart, so only the block count fails)
    (dict(S=8193 * 64, gt=8193, gh=64, gw=1, xq=ctypes.c_void_p(1 << 32), xk=ctypes.c_void_p(2 << 32),
          q_out=ctypes.c_void_p(3 << 32), k_out=ctypes.c_void_p(4 << 32)), 2),
])
def test_norm_rope_select_rejects_bad_arguments(args, status):
    a = dict(xq=ctypes.c_void_p(0x10000), xk=ctypes.c_void_p(0x100000), wq=ctypes.c_void_p(0x20000),
             wk=ctypes.c_void_p(0x30000), B=1, H=4, S=12, D=128, block=64, gt=1, gh=3, gw=4, eps=1e-6, theta=1e4,
             r=0.5, q_out=ctypes.c_void_p(0x1000000), k_out=ctypes.c_void_p(0x2000000), rp=FAKE, ci=FAKE, ws=FAKE,
             ws_bytes=1 << 30)
    a.update(args)
    st = lib().bsa_norm_rope_select(a["xq"], a["xk"], a["wq"], a["wk"], a["B"], a["H"], a["S"], a["D"], a["block"],
                                    a["gt"], a["gh"], a["gw"], a["eps"], a["theta"], a["r"], a["q_out"], a["k_out"],
                                    a["rp"], a["ci"], a["ws"], a["ws_bytes"], None)
    assert st == status, bsa.bsa_last_error()


def test_binding_fails_loudly_without_the_library(tmp_path):
    """With libbsa.so absent the package raises ImportError on first use: there is no CPU or
    PyTorch fallback."""
    import subprocess
    import sys

    pkg = os.path.join(ROOT, "dynamic_block_sparse_bsa_amd", "__init__.py")
    code = ("import importlib.util, sys\n"
            "spec = importlib.util.spec_from_file_location('bsa_copy', %r)\n"
            "m = importlib.util.module_from_spec(spec); spec.loader.exec_module(m)\n"
            "m.lib_path = %r\n"
            "try:\n    m.bsa_num_blocks(10, 4)\nexcept ImportError as e:\n    print('IMPORT_ERROR', e); sys.exit(0)\n"
            "sys.exit(1)\n") % (pkg, str(tmp_path / "missing" / "libbsa.so"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "IMPORT_ERROR" in r.stdout, r.stdout + r.stderr


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys

    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
