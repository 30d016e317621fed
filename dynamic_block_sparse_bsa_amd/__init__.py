"""Dynamic block-sparse self-attention for AMD Instinct MI355X (gfx950).

Thin Python binding over libbsa.so, the C-ABI library declared in include/bsa.h. This
module only marshals arguments: torch provides device memory and the current stream,
and every step of the computation runs in libbsa's HIP kernels. There is no CPU or
PyTorch fallback: if libbsa.so is missing or a call fails, an exception is raised.

Function names match the C entry points. Tensors are contiguous [B, H, S, D] on a HIP
device: bf16 for q, k, v and outputs, uint8 (E4M3FN bit patterns) for fp8 codes.
"""
import ctypes
import os

import torch

__all__ = [
    "BsaError", "lib_path", "bsa_num_blocks", "bsa_num_kept", "bsa_select_workspace_bytes",
    "bsa_pool", "bsa_select", "bsa_select_noalloc", "bsa_select_noalloc_max_bytes", "bsa_forward", "bsa_quantize_fp8", "bsa_forward_fp8",
    "bsa_check_csr", "bsa_status_string", "bsa_last_error", "bsa_vt_fp8_bytes", "bsa_select_quantize",
    "bsa_quantize_v_fp8", "bsa_forward_fp8_full", "bsa_norm_rope_workspace_bytes", "bsa_norm_rope",
    "bsa_norm_rope_select_workspace_bytes", "bsa_norm_rope_select",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libbsa.so")

BSA_OK = 0
STATUS_NAMES = {0: "BSA_OK", 1: "BSA_ERR_INVALID_ARGUMENT", 2: "BSA_ERR_UNSUPPORTED",
                3: "BSA_ERR_WORKSPACE_TOO_SMALL", 4: "BSA_ERR_NO_DEVICE", 5: "BSA_ERR_HIP"}


class BsaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, str(status)), message))
        self.status = status


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise ImportError("libbsa.so is not built (expected at %s); run __graft_entry__.build()" % lib_path)
    lib = ctypes.CDLL(lib_path)
    P, i32, f64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double, ctypes.c_size_t
    sig = {
        "bsa_num_blocks": (i32, [i32, i32]),
        "bsa_num_kept": (i32, [i32, f64]),
        "bsa_select_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "bsa_pool": (ctypes.c_int, [P, i32, i32, i32, i32, i32, P, P]),
        "bsa_select": (ctypes.c_int, [P, P, i32, i32, i32, i32, i32, f64, P, P, P, sz, P]),
        "bsa_select_noalloc": (ctypes.c_int, [P, P, i32, i32, i32, i32, i32, f64, P, P, P]),
        "bsa_select_noalloc_max_bytes": (sz, []),
        "bsa_forward": (ctypes.c_int, [P, P, P, i32, i32, i32, i32, i32, P, P, P, P]),
        "bsa_quantize_fp8": (ctypes.c_int, [P, i32, i32, i32, i32, i32, P, P, P]),
        "bsa_forward_fp8": (ctypes.c_int, [P, P, P, P, P, i32, i32, i32, i32, i32, P, P, P, P]),
        "bsa_check_csr": (ctypes.c_int, [P, ctypes.c_int64, P, ctypes.c_int64, i32, i32]),
        "bsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "bsa_last_error": (ctypes.c_char_p, []),
        "bsa_vt_fp8_bytes": (sz, [i32, i32, i32, i32, i32]),
        "bsa_select_quantize": (ctypes.c_int, [P, P, i32, i32, i32, i32, i32, f64, P, P, P, P, P, P, P, sz, P]),
        "bsa_quantize_v_fp8": (ctypes.c_int, [P, i32, i32, i32, i32, i32, P, P, P]),
        "bsa_forward_fp8_full": (ctypes.c_int, [P, P, P, P, P, P, i32, i32, i32, i32, i32, P, P, P, P]),
        "bsa_norm_rope_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "bsa_norm_rope": (ctypes.c_int, [P, P, i32, i32, i32, i32, i32, i32, i32, i32, f64, f64, P, P, P, sz, P]),
        "bsa_norm_rope_select_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "bsa_norm_rope_select": (ctypes.c_int, [P, P, P, P, i32, i32, i32, i32, i32, i32, i32, i32, f64, f64, f64,
                                                P, P, P, P, P, sz, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(status):
    if status != BSA_OK:
        raise BsaError(status, _load().bsa_last_error().decode())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev_tensor(t, name, dtypes, ndim=4):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a HIP device (got %s)" % (name, t.device))
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dimensions" % (name, ndim))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


_ONE_BYTE = (torch.uint8, torch.int8, torch.float8_e4m3fn)


def _given(t, name, dtypes, numel, device, shape=None):
    """Checks a caller-provided output or buffer before any launch: a contiguous tensor on
    `device` of one of `dtypes` with exactly `numel` elements (and `shape`, if given)."""
    _dev_tensor(t, name, dtypes, ndim=None)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.numel() != numel:
        raise ValueError("%s has %d elements, expected %d" % (name, t.numel(), numel))
    return t


def _bytes_at_least(t, name, nbytes, device):
    """A caller's scratch buffer: any dtype, contiguous, on `device`, at least nbytes."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    _dev_tensor(t, name, (t.dtype,), ndim=None)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.numel() * t.element_size() < nbytes:
        raise ValueError("%s holds %d bytes, needs %d" % (name, t.numel() * t.element_size(), nbytes))
    return t


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def bsa_num_blocks(S: int, block: int) -> int:
    return _load().bsa_num_blocks(S, block)


def bsa_num_kept(n_blocks: int, keep_ratio: float) -> int:
    return _load().bsa_num_kept(n_blocks, keep_ratio)


def bsa_select_workspace_bytes(B, H, S, D, block) -> int:
    return _load().bsa_select_workspace_bytes(B, H, S, D, block)


def bsa_pool(x, block: int, out=None):
    """fp32 block means [B, H, n, D] of a bf16 [B, H, S, D] tensor."""
    _dev_tensor(x, "x", (torch.bfloat16,))
    B, H, S, D = x.shape
    n = bsa_num_blocks(S, block)
    if out is None:
        out = torch.empty((B, H, n, D), dtype=torch.float32, device=x.device)
    _given(out, "out", (torch.float32,), B * H * n * D, x.device)
    _check(_load().bsa_pool(_p(x), B, H, S, D, block, _p(out), _stream(x)))
    return out


def bsa_select(q, k, block: int, keep_ratio: float, workspace=None, row_ptr=None, col_idx=None):
    """Kept key-block lists (row_ptr int32 [B*H*n+1], col_idx int32 [B*H*n*kept])."""
    _dev_tensor(q, "q", (torch.bfloat16,))
    _dev_tensor(k, "k", (torch.bfloat16,))
    if q.shape != k.shape:
        raise ValueError("q and k shapes differ")
    B, H, S, D = q.shape
    n = bsa_num_blocks(S, block)
    kept = bsa_num_kept(n, keep_ratio)
    if kept == 0:
        raise BsaError(1, "keep_ratio must be in (0, 1] (got %r)" % (keep_ratio,))
    rows = B * H * n
    ws_bytes = bsa_select_workspace_bytes(B, H, S, D, block)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    if row_ptr is None:
        row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=q.device)
    if col_idx is None:
        col_idx = torch.empty(rows * kept, dtype=torch.int32, device=q.device)
    _bytes_at_least(workspace, "workspace", ws_bytes, q.device)
    _given(row_ptr, "row_ptr", (torch.int32,), rows + 1, q.device)
    _given(col_idx, "col_idx", (torch.int32,), rows * kept, q.device)
    _check(_load().bsa_select(_p(q), _p(k), B, H, S, D, block, keep_ratio, _p(row_ptr), _p(col_idx),
                              _p(workspace), workspace.numel() * workspace.element_size(), _stream(q)))
    return row_ptr, col_idx


def bsa_select_noalloc_max_bytes() -> int:
    return _load().bsa_select_noalloc_max_bytes()


def bsa_select_noalloc(q, k, block: int, keep_ratio: float, row_ptr=None, col_idx=None):
    """bsa_select with the block means in the library's own scratch array: the C call
    allocates nothing (pass row_ptr and col_idx to keep this function allocation-free too)."""
    _dev_tensor(q, "q", (torch.bfloat16,))
    _dev_tensor(k, "k", (torch.bfloat16,))
    if q.shape != k.shape:
        raise ValueError("q and k shapes differ")
    B, H, S, D = q.shape
    n = bsa_num_blocks(S, block)
    kept = bsa_num_kept(n, keep_ratio)
    if kept == 0:
        raise BsaError(1, "keep_ratio must be in (0, 1] (got %r)" % (keep_ratio,))
    rows = B * H * n
    if row_ptr is None:
        row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=q.device)
    if col_idx is None:
        col_idx = torch.empty(rows * kept, dtype=torch.int32, device=q.device)
    _given(row_ptr, "row_ptr", (torch.int32,), rows + 1, q.device)
    _given(col_idx, "col_idx", (torch.int32,), rows * kept, q.device)
    _check(_load().bsa_select_noalloc(_p(q), _p(k), B, H, S, D, block, keep_ratio, _p(row_ptr), _p(col_idx),
                                      _stream(q)))
    return row_ptr, col_idx


def _csr(row_ptr, col_idx, device, rows):
    """Device CSR over `rows` query-block rows. col_idx must hold row_ptr[rows] entries; that
    count lives on the device and is not read here (reading it would synchronise)."""
    for t, name in ((row_ptr, "row_ptr"), (col_idx, "col_idx")):
        _dev_tensor(t, name, (torch.int32,), ndim=1)
        if t.device != device:
            raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if row_ptr.numel() != rows + 1:
        raise ValueError("row_ptr has %d entries, expected B*H*n + 1 = %d" % (row_ptr.numel(), rows + 1))


def bsa_forward(q, k, v, block: int, row_ptr, col_idx, out=None):
    """Attention over the kept blocks; bf16 [B, H, S, D]."""
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _dev_tensor(t, name, (torch.bfloat16,))
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v shapes differ")
    B, H, S, D = q.shape
    _csr(row_ptr, col_idx, q.device, B * H * bsa_num_blocks(S, block))
    if out is None:
        out = torch.empty_like(q)
    _given(out, "out", (torch.bfloat16,), q.numel(), q.device, shape=q.shape)
    _check(_load().bsa_forward(_p(q), _p(k), _p(v), B, H, S, D, block, _p(row_ptr), _p(col_idx), _p(out),
                               _stream(q)))
    return out


def bsa_quantize_fp8(x, block: int, codes=None, scale=None):
    """(codes uint8 [B,H,S,D] holding E4M3FN, scale fp32 [B,H,n]) per token block."""
    _dev_tensor(x, "x", (torch.bfloat16,))
    B, H, S, D = x.shape
    n = bsa_num_blocks(S, block)
    if codes is None:
        codes = torch.empty((B, H, S, D), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((B, H, n), dtype=torch.float32, device=x.device)
    _given(codes, "codes", _ONE_BYTE, x.numel(), x.device)
    _given(scale, "scale", (torch.float32,), B * H * n, x.device)
    _check(_load().bsa_quantize_fp8(_p(x), B, H, S, D, block, _p(codes), _p(scale), _stream(x)))
    return codes, scale


def bsa_forward_fp8(q8, q_scale, k8, k_scale, v, block: int, row_ptr, col_idx, out=None):
    """Attention with E4M3FN Q/K codes and per-block scales, bf16 V; bf16 output."""
    _dev_tensor(q8, "q_e4m3", _ONE_BYTE)
    _dev_tensor(k8, "k_e4m3", _ONE_BYTE)
    _dev_tensor(v, "v", (torch.bfloat16,))
    if not (q8.shape == k8.shape == v.shape):
        raise ValueError("q_e4m3, k_e4m3 and v shapes differ")
    B, H, S, D = v.shape
    n = bsa_num_blocks(S, block)
    for t, name in ((q_scale, "q_scale"), (k_scale, "k_scale")):
        _dev_tensor(t, name, (torch.float32,), ndim=None)
        if t.numel() != B * H * n:
            raise ValueError("%s must have B*H*n = %d entries" % (name, B * H * n))
    _csr(row_ptr, col_idx, v.device, B * H * n)
    for t, name in ((q8, "q_e4m3"), (k8, "k_e4m3"), (q_scale, "q_scale"), (k_scale, "k_scale")):
        if t.device != v.device:
            raise ValueError("%s is on %s, expected %s" % (name, t.device, v.device))
    if out is None:
        out = torch.empty_like(v)
    _given(out, "out", (torch.bfloat16,), v.numel(), v.device, shape=v.shape)
    _check(_load().bsa_forward_fp8(_p(q8), _p(q_scale), _p(k8), _p(k_scale), _p(v), B, H, S, D, block,
                                   _p(row_ptr), _p(col_idx), _p(out), _stream(v)))
    return out


def bsa_vt_fp8_bytes(B, H, S, D, block) -> int:
    return _load().bsa_vt_fp8_bytes(B, H, S, D, block)


def bsa_select_quantize(q, k, block: int, keep_ratio: float, workspace=None, row_ptr=None, col_idx=None):
    """(row_ptr, col_idx, q_codes, q_scale, k_codes, k_scale): bsa_select's lists and the
    per-block E4M3 codes and scales of q and k, from one read of each block."""
    _dev_tensor(q, "q", (torch.bfloat16,))
    _dev_tensor(k, "k", (torch.bfloat16,))
    if q.shape != k.shape:
        raise ValueError("q and k shapes differ")
    B, H, S, D = q.shape
    n = bsa_num_blocks(S, block)
    kept = bsa_num_kept(n, keep_ratio)
    if kept == 0:
        raise BsaError(1, "keep_ratio must be in (0, 1] (got %r)" % (keep_ratio,))
    rows = B * H * n
    if workspace is None:
        workspace = torch.empty(max(bsa_select_workspace_bytes(B, H, S, D, block), 1), dtype=torch.uint8, device=q.device)
    if row_ptr is None:
        row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=q.device)
    if col_idx is None:
        col_idx = torch.empty(rows * kept, dtype=torch.int32, device=q.device)
    _bytes_at_least(workspace, "workspace", bsa_select_workspace_bytes(B, H, S, D, block), q.device)
    _given(row_ptr, "row_ptr", (torch.int32,), rows + 1, q.device)
    _given(col_idx, "col_idx", (torch.int32,), rows * kept, q.device)
    q8 = torch.empty((B, H, S, D), dtype=torch.uint8, device=q.device)
    k8 = torch.empty_like(q8)
    qs = torch.empty((B, H, n), dtype=torch.float32, device=q.device)
    ks = torch.empty_like(qs)
    _check(_load().bsa_select_quantize(_p(q), _p(k), B, H, S, D, block, keep_ratio, _p(row_ptr), _p(col_idx), _p(q8),
                                       _p(qs), _p(k8), _p(ks), _p(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(q)))
    return row_ptr, col_idx, q8, qs, k8, ks


def bsa_quantize_v_fp8(v, block: int, vt=None, scale=None):
    """(vt uint8 [B*H, D, ceil(S/block)*block] transposed, key-permuted E4M3 codes,
    scale fp32 [B, H, D]) per (batch, head, channel)."""
    _dev_tensor(v, "v", (torch.bfloat16,))
    B, H, S, D = v.shape
    n = bsa_num_blocks(S, block)
    if vt is None:
        vt = torch.empty((B * H, D, n * block), dtype=torch.uint8, device=v.device)
    if scale is None:
        scale = torch.empty((B, H, D), dtype=torch.float32, device=v.device)
    _given(vt, "vt", _ONE_BYTE, bsa_vt_fp8_bytes(B, H, S, D, block), v.device)
    _given(scale, "scale", (torch.float32,), B * H * D, v.device)
    _check(_load().bsa_quantize_v_fp8(_p(v), B, H, S, D, block, _p(vt), _p(scale), _stream(v)))
    return vt, scale


def bsa_forward_fp8_full(q8, q_scale, k8, k_scale, vt8, v_scale, block: int, row_ptr, col_idx, out=None):
    """Attention with E4M3 Q, K, V and E4M3 softmax weights; bf16 output [B, H, S, D]."""
    _dev_tensor(q8, "q_e4m3", _ONE_BYTE)
    _dev_tensor(k8, "k_e4m3", _ONE_BYTE)
    _dev_tensor(vt8, "vt_e4m3", _ONE_BYTE, ndim=None)
    if q8.shape != k8.shape:
        raise ValueError("q_e4m3 and k_e4m3 shapes differ")
    B, H, S, D = q8.shape
    n = bsa_num_blocks(S, block)
    if vt8.numel() != bsa_vt_fp8_bytes(B, H, S, D, block):
        raise ValueError("vt_e4m3 must hold bsa_vt_fp8_bytes bytes for this shape and block")
    for t, name, cnt in ((q_scale, "q_scale", B * H * n), (k_scale, "k_scale", B * H * n), (v_scale, "v_scale", B * H * D)):
        _dev_tensor(t, name, (torch.float32,), ndim=None)
        if t.numel() != cnt:
            raise ValueError("%s must have %d entries" % (name, cnt))
    _csr(row_ptr, col_idx, q8.device, B * H * n)
    for t, name in ((k8, "k_e4m3"), (vt8, "vt_e4m3"), (q_scale, "q_scale"), (k_scale, "k_scale"), (v_scale, "v_scale")):
        if t.device != q8.device:
            raise ValueError("%s is on %s, expected %s" % (name, t.device, q8.device))
    if out is None:
        out = torch.empty((B, H, S, D), dtype=torch.bfloat16, device=q8.device)
    _given(out, "out", (torch.bfloat16,), B * H * S * D, q8.device, shape=(B, H, S, D))
    _check(_load().bsa_forward_fp8_full(_p(q8), _p(q_scale), _p(k8), _p(k_scale), _p(vt8), _p(v_scale), B, H, S, D,
                                        block, _p(row_ptr), _p(col_idx), _p(out), _stream(q8)))
    return out


def bsa_check_csr(row_ptr, col_idx, rows: int, n_blocks: int):
    """Validate a host-side CSR (numpy or CPU tensors); raises BsaError on a violation."""
    import numpy as np
    rp = np.ascontiguousarray(row_ptr, dtype=np.int32).reshape(-1)
    ci = np.ascontiguousarray(col_idx, dtype=np.int32).reshape(-1)
    _check(_load().bsa_check_csr(ctypes.c_void_p(rp.ctypes.data), rp.size, ctypes.c_void_p(ci.ctypes.data), ci.size,
                                 rows, n_blocks))


def bsa_status_string(status: int) -> str:
    return _load().bsa_status_string(status).decode()


def bsa_last_error() -> str:
    return _load().bsa_last_error().decode()


def bsa_norm_rope_workspace_bytes(B, H, S, D) -> int:
    return _load().bsa_norm_rope_workspace_bytes(B, H, S, D)


def bsa_norm_rope_select_workspace_bytes(B, H, S, D, block) -> int:
    return _load().bsa_norm_rope_select_workspace_bytes(B, H, S, D, block)


def _projection(x, w, name):
    _dev_tensor(x, name, (torch.bfloat16,))
    _dev_tensor(w, "w" + name[1:], (torch.bfloat16,), ndim=1)
    B, S, H, D = x.shape
    if w.numel() != H * D:
        raise ValueError("%s must hold H*D = %d weights" % ("w" + name[1:], H * D))
    return B, S, H, D


def bsa_norm_rope(x, weight, block: int, grid, eps: float = 1e-6, theta: float = 10000.0, means: bool = True,
                  out=None, xbar=None, workspace=None):
    """RMSNorm over each token's H*D channels, 3D RoPE per head, written head-major.

    x: bf16 [B, S, H, D] (a projection's output viewed per head, token-major); weight: bf16
    [H*D]; grid: (Gt, Gh, Gw) with Gt*Gh*Gw = S. Returns out bf16 [B, H, S, D] and, if
    means, the fp32 block means [B, H, n, D] of out (else None)."""
    B, S, H, D = _projection(x, weight, "x")
    gt, gh, gw = (int(g) for g in grid)
    if out is None:
        out = torch.empty((B, H, S, D), dtype=torch.bfloat16, device=x.device)
    _given(out, "out", (torch.bfloat16,), B * H * S * D, x.device, shape=(B, H, S, D))
    ws_bytes = 0
    if means:
        n = bsa_num_blocks(S, block)
        if xbar is None:
            xbar = torch.empty((B, H, n, D), dtype=torch.float32, device=x.device)
        _given(xbar, "xbar", (torch.float32,), B * H * n * D, x.device)
        ws_bytes = bsa_norm_rope_workspace_bytes(B, H, S, D)
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
        _bytes_at_least(workspace, "workspace", ws_bytes, x.device)
    else:
        xbar = None
    _check(_load().bsa_norm_rope(_p(x), _p(weight), B, H, S, D, block, gt, gh, gw, float(eps), float(theta), _p(out),
                                 _p(xbar) if xbar is not None else None,
                                 _p(workspace) if workspace is not None else None,
                                 workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                 _stream(x)))
    return out, xbar


def bsa_norm_rope_select(xq, xk, wq, wk, block: int, grid, keep_ratio: float, eps: float = 1e-6,
                         theta: float = 10000.0, workspace=None):
    """bsa_norm_rope of both projections and bsa_select's lists from the fused means:
    returns (q bf16 [B, H, S, D], k bf16 [B, H, S, D], row_ptr, col_idx)."""
    B, S, H, D = _projection(xq, wq, "xq")
    if _projection(xk, wk, "xk") != (B, S, H, D):
        raise ValueError("xq and xk shapes differ")
    gt, gh, gw = (int(g) for g in grid)
    n = bsa_num_blocks(S, block)
    kept = bsa_num_kept(n, keep_ratio)
    if kept == 0:
        raise BsaError(1, "keep_ratio must be in (0, 1] (got %r)" % (keep_ratio,))
    q = torch.empty((B, H, S, D), dtype=torch.bfloat16, device=xq.device)
    k = torch.empty_like(q)
    rows = B * H * n
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=xq.device)
    col_idx = torch.empty(rows * kept, dtype=torch.int32, device=xq.device)
    ws_bytes = bsa_norm_rope_select_workspace_bytes(B, H, S, D, block)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=xq.device)
    _bytes_at_least(workspace, "workspace", ws_bytes, xq.device)
    _check(_load().bsa_norm_rope_select(_p(xq), _p(xk), _p(wq), _p(wk), B, H, S, D, block, gt, gh, gw, float(eps),
                                        float(theta), float(keep_ratio), _p(q), _p(k), _p(row_ptr), _p(col_idx),
                                        _p(workspace), workspace.numel() * workspace.element_size(), _stream(xq)))
    return q, k, row_ptr, col_idx
