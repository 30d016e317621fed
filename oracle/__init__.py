"""CPU oracle for dynamic block-sparse self-attention.

TEST INFRASTRUCTURE ONLY. Only tests/, the smoke check in __graft_entry__.py and the
CPU-baseline leg of bench.py may import this package. The GPU library never does, and
nothing here is derived from the GPU library: the arithmetic lives in bsa_oracle.c
(plain C, fp64), which follows the pages' description of the method:

* "知识卡片：600倍加速，720p视频实时生成！单卡也能带的动14B模型" (ai.cheesepanini.fun
  knowledge card), section 方法/产品要点, item 动态稀疏量化注意力 -- block means of Q and
  K estimate attention importance; only the activated key blocks are computed; about
  10-20 % of blocks are kept; an FP8 path via SageAttention2.
* "单卡 RTX 5090 跑 Wan2.2-A14B：720p 视频生成只要 3.8 秒" (aoyii.com), section
  四步拆解, step 3 动态稀疏注意力 -- the computation inside selected blocks stays dense.

This module only marshals numpy arrays to the C functions and checks their shapes.
bf16 tensors are numpy uint16 arrays holding the raw bf16 bit patterns, shaped
[B, H, S, D]. Every function here is pinned by tests/test_oracle_pins.py.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("BSA_ORACLE_LIB")  # another build of bsa_oracle.c (mutation tests)
    if not path:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
    _lib = _bind(ctypes.CDLL(path))
    return _lib


class use_library:
    """Context manager: route every call of this module to another build of bsa_oracle.c
    (the mutation tests load deliberately broken copies through it)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _load()
        _lib = _bind(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _bind(lib):
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_num_blocks.restype = i32
    lib.oracle_num_blocks.argtypes = [i32, i32]
    lib.oracle_num_kept.restype = i32
    lib.oracle_num_kept.argtypes = [i32, f64]
    lib.oracle_e4m3_value.restype = f64
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode.argtypes = [f64]
    lib.oracle_pool.restype = None
    lib.oracle_pool.argtypes = [P, i32, i32, i32, i32, i32, P]
    lib.oracle_scores.restype = None
    lib.oracle_scores.argtypes = [P, P, i32, i32, i32, P]
    lib.oracle_select.restype = None
    lib.oracle_select.argtypes = [P, i32, i32, i32, P, P]
    lib.oracle_attention.restype = None
    lib.oracle_attention.argtypes = [P, P, P, i32, i32, i32, i32, i32, P, P, P, i64, P]
    lib.oracle_quantize_fp8.restype = None
    lib.oracle_quantize_fp8.argtypes = [P, i32, i32, i32, i32, i32, P, P]
    lib.oracle_attention_fp8.restype = None
    lib.oracle_attention_fp8.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, P, P, P, i64, P]
    lib.oracle_quantize_v_fp8.restype = None
    lib.oracle_quantize_v_fp8.argtypes = [P, i32, i32, i32, i32, P, P]
    lib.oracle_attention_fp8_qkv.restype = None
    lib.oracle_attention_fp8_qkv.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, P, P, P, i64, P, P]
    lib.oracle_attention_fp8_full.restype = None
    lib.oracle_attention_fp8_full.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, P, P, P, i64, P]
    lib.oracle_round_bf16.restype = ctypes.c_uint16
    lib.oracle_round_bf16.argtypes = [f64]
    lib.oracle_norm_rope.restype = None
    lib.oracle_norm_rope.argtypes = [P, P, i32, i32, i32, i32, i32, i32, i32, f64, f64, P, P]
    return lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _bf16_tensor(x):
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16 or x.ndim != 4:
        raise ValueError("expected a [B, H, S, D] uint16 array of bf16 bit patterns")
    return x


def num_blocks(S: int, block: int) -> int:
    return _load().oracle_num_blocks(S, block)


def num_kept(n: int, keep_ratio: float) -> int:
    return _load().oracle_num_kept(n, keep_ratio)


def e4m3_value(code: int) -> float:
    return _load().oracle_e4m3_value(code)


def e4m3_encode(x: float) -> int:
    return _load().oracle_e4m3_encode(x)


def pool(x, block: int) -> np.ndarray:
    """Block means [B, H, n, D] (fp64) of a bf16 tensor."""
    x = _bf16_tensor(x)
    B, H, S, D = x.shape
    n = num_blocks(S, block)
    out = np.empty((B, H, n, D), dtype=np.float64)
    _load().oracle_pool(_ptr(x), B, H, S, D, block, _ptr(out))
    return out


def scores(qbar, kbar) -> np.ndarray:
    """Block-pair scores [B, H, n, n] = qbar . kbar / sqrt(D), fp64."""
    qbar = np.ascontiguousarray(qbar, dtype=np.float64)
    kbar = np.ascontiguousarray(kbar, dtype=np.float64)
    B, H, n, D = qbar.shape
    if kbar.shape != qbar.shape:
        raise ValueError("qbar and kbar shapes differ")
    out = np.empty((B, H, n, n), dtype=np.float64)
    _load().oracle_scores(_ptr(qbar), _ptr(kbar), B * H, n, D, _ptr(out))
    return out


def select_from_scores(s, k: int):
    """Top-k of each row of s [B, H, n, n] by (score desc, index asc), emitted ascending.

    Returns (row_ptr int32 [B*H*n+1], col_idx int32 [B*H*n*k], gap fp64 [B*H*n]) where gap
    is the k-th minus the (k+1)-th largest score of the row (+inf when k = n)."""
    s = np.ascontiguousarray(s, dtype=np.float64)
    B, H, n, n2 = s.shape
    if n != n2 or not (1 <= k <= n):
        raise ValueError("bad score shape or k")
    rows = B * H * n
    col = np.empty(rows * k, dtype=np.int32)
    gap = np.empty(rows, dtype=np.float64)
    _load().oracle_select(_ptr(s), rows, n, k, _ptr(col), _ptr(gap))
    row_ptr = (np.arange(rows + 1, dtype=np.int64) * k).astype(np.int32)
    return row_ptr, col, gap


def select(q, k, block: int, keep_ratio: float):
    """The whole selection: pool Q and K, score block pairs, keep the top k per row.

    Returns dict(row_ptr, col_idx, gap, scores, kept)."""
    q = _bf16_tensor(q)
    k = _bf16_tensor(k)
    B, H, S, D = q.shape
    n = num_blocks(S, block)
    kept = num_kept(n, keep_ratio)
    if kept == 0:
        raise ValueError("invalid keep_ratio")
    s = scores(pool(q, block), pool(k, block))
    row_ptr, col, gap = select_from_scores(s, kept)
    return {"row_ptr": row_ptr, "col_idx": col, "gap": gap, "scores": s, "kept": kept}


def check_csr(row_ptr, col_idx, rows: int, n: int):
    row_ptr = np.asarray(row_ptr)
    col_idx = np.asarray(col_idx)
    if row_ptr.shape != (rows + 1,) or row_ptr[0] != 0 or np.any(np.diff(row_ptr) < 0):
        raise ValueError("malformed row_ptr")
    if row_ptr[-1] > col_idx.size:
        raise ValueError("col_idx shorter than row_ptr[-1]")
    for r in range(rows):
        c = col_idx[row_ptr[r]:row_ptr[r + 1]]
        if c.size and (c[0] < 0 or c[-1] >= n or np.any(np.diff(c) <= 0)):
            raise ValueError("row %d: indices must be strictly ascending in [0, n)" % r)


def _tokens_arg(tokens):
    if tokens is None:
        return None, 0
    t = np.ascontiguousarray(tokens, dtype=np.int64)
    return t, t.size


def attention(q, k, v, block: int, row_ptr, col_idx, tokens=None) -> np.ndarray:
    """fp64 block-sparse attention. tokens: flat query indices (b*H+h)*S+t, or None for all.

    Returns [len(tokens), D], or [B, H, S, D] when tokens is None."""
    q, k, v = _bf16_tensor(q), _bf16_tensor(k), _bf16_tensor(v)
    B, H, S, D = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v shapes differ")
    n = num_blocks(S, block)
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col_idx = np.ascontiguousarray(col_idx, dtype=np.int32)
    check_csr(row_ptr, col_idx, B * H * n, n)
    t, nt = _tokens_arg(tokens)
    if t is not None and (np.any(t < 0) or np.any(t >= B * H * S)):
        raise ValueError("token index out of range")
    out = np.empty(((B * H * S) if t is None else nt, D), dtype=np.float64)
    _load().oracle_attention(_ptr(q), _ptr(k), _ptr(v), B, H, S, D, block, _ptr(row_ptr),
                             _ptr(col_idx), _ptr(t), nt, _ptr(out))
    return out.reshape(B, H, S, D) if t is None else out


def quantize_fp8(x, block: int):
    """(codes uint8 [B,H,S,D], scale float32 [B,H,n]) per (batch, head, token block)."""
    x = _bf16_tensor(x)
    B, H, S, D = x.shape
    n = num_blocks(S, block)
    codes = np.empty((B, H, S, D), dtype=np.uint8)
    scale = np.empty((B, H, n), dtype=np.float32)
    _load().oracle_quantize_fp8(_ptr(x), B, H, S, D, block, _ptr(codes), _ptr(scale))
    return codes, scale


def attention_fp8(q8, q_scale, k8, k_scale, v, block: int, row_ptr, col_idx, tokens=None):
    """Attention with Q, K dequantised from E4M3 codes and per-block scales; V bf16."""
    v = _bf16_tensor(v)
    B, H, S, D = v.shape
    n = num_blocks(S, block)
    q8 = np.ascontiguousarray(q8, dtype=np.uint8)
    k8 = np.ascontiguousarray(k8, dtype=np.uint8)
    q_scale = np.ascontiguousarray(q_scale, dtype=np.float32)
    k_scale = np.ascontiguousarray(k_scale, dtype=np.float32)
    if q8.shape != v.shape or k8.shape != v.shape or q_scale.size != B * H * n or k_scale.size != B * H * n:
        raise ValueError("fp8 operand shapes do not match")
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col_idx = np.ascontiguousarray(col_idx, dtype=np.int32)
    check_csr(row_ptr, col_idx, B * H * n, n)
    t, nt = _tokens_arg(tokens)
    out = np.empty(((B * H * S) if t is None else nt, D), dtype=np.float64)
    _load().oracle_attention_fp8(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(v), B, H,
                                 S, D, block, _ptr(row_ptr), _ptr(col_idx), _ptr(t), nt, _ptr(out))
    return out.reshape(B, H, S, D) if t is None else out


def quantize_v_fp8(v):
    """(codes uint8 [B,H,S,D], scale float32 [B,H,D]): one scale per (batch, head, channel)
    over the whole sequence, the full FP8 path's reading for V."""
    v = _bf16_tensor(v)
    B, H, S, D = v.shape
    codes = np.empty((B, H, S, D), dtype=np.uint8)
    scale = np.empty((B, H, D), dtype=np.float32)
    _load().oracle_quantize_v_fp8(_ptr(v), B, H, S, D, _ptr(codes), _ptr(scale))
    return codes, scale


def attention_fp8_qkv(q8, q_scale, k8, k_scale, v8, v_scale, block: int, row_ptr, col_idx, tokens=None,
                      spread=False):
    """Exact (fp64) attention over the full FP8 path's dequantised operands: Q, K with
    per-block scales, V with per-channel scales (codes in the [B, H, S, D] layout of
    quantize_v_fp8); the softmax weights are not rounded. With spread=True also returns
    dev [..., 3, D]: sum_u p_u |v_u - o|, sum_u |v_u - o| and sqrt(sum_u p_u^2 (v_u - o)^2)."""
    q8 = np.ascontiguousarray(q8, dtype=np.uint8)
    k8 = np.ascontiguousarray(k8, dtype=np.uint8)
    v8 = np.ascontiguousarray(v8, dtype=np.uint8)
    if q8.ndim != 4 or k8.shape != q8.shape or v8.shape != q8.shape:
        raise ValueError("fp8 operand shapes do not match")
    B, H, S, D = q8.shape
    n = num_blocks(S, block)
    q_scale = np.ascontiguousarray(q_scale, dtype=np.float32)
    k_scale = np.ascontiguousarray(k_scale, dtype=np.float32)
    v_scale = np.ascontiguousarray(v_scale, dtype=np.float32)
    if q_scale.size != B * H * n or k_scale.size != B * H * n or v_scale.size != B * H * D:
        raise ValueError("scale shapes do not match")
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col_idx = np.ascontiguousarray(col_idx, dtype=np.int32)
    check_csr(row_ptr, col_idx, B * H * n, n)
    t, nt = _tokens_arg(tokens)
    rows = (B * H * S) if t is None else nt
    out = np.empty((rows, D), dtype=np.float64)
    dev = np.empty((rows, 3, D), dtype=np.float64) if spread else None
    _load().oracle_attention_fp8_qkv(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(v8), _ptr(v_scale),
                                     B, H, S, D, block, _ptr(row_ptr), _ptr(col_idx), _ptr(t), nt, _ptr(out),
                                     _ptr(dev))
    if t is None:
        out = out.reshape(B, H, S, D)
        dev = dev.reshape(B, H, S, 3, D) if spread else None
    return (out, dev) if spread else out


def attention_fp8_full(q8, q_scale, k8, k_scale, v8, v_scale, block: int, row_ptr, col_idx, tokens=None):
    """The full FP8 path: Q, K (per-block scales) and V (per-channel scales) as E4M3 codes,
    online softmax over 64-key sub-tiles in list order with the weights stored as E4M3."""
    q8 = np.ascontiguousarray(q8, dtype=np.uint8)
    k8 = np.ascontiguousarray(k8, dtype=np.uint8)
    v8 = np.ascontiguousarray(v8, dtype=np.uint8)
    if q8.ndim != 4 or k8.shape != q8.shape or v8.shape != q8.shape:
        raise ValueError("fp8 operand shapes do not match")
    B, H, S, D = q8.shape
    n = num_blocks(S, block)
    q_scale = np.ascontiguousarray(q_scale, dtype=np.float32)
    k_scale = np.ascontiguousarray(k_scale, dtype=np.float32)
    v_scale = np.ascontiguousarray(v_scale, dtype=np.float32)
    if q_scale.size != B * H * n or k_scale.size != B * H * n or v_scale.size != B * H * D:
        raise ValueError("scale shapes do not match")
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col_idx = np.ascontiguousarray(col_idx, dtype=np.int32)
    if row_ptr.size != B * H * n + 1 or row_ptr[-1] > col_idx.size:
        raise ValueError("row_ptr / col_idx do not describe B*H*n rows")
    t, nt = _tokens_arg(tokens)
    out = np.empty(((B * H * S) if t is None else nt, D), dtype=np.float64)
    _load().oracle_attention_fp8_full(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(v8), _ptr(v_scale),
                                      B, H, S, D, block, _ptr(row_ptr), _ptr(col_idx), _ptr(t), nt, _ptr(out))
    return out.reshape(B, H, S, D) if t is None else out


def round_bf16(x: float) -> int:
    """Bit pattern of the bf16 nearest to x (ties to even)."""
    return _load().oracle_round_bf16(float(x))


def norm_rope(x, w, grid, eps: float = 1e-6, theta: float = 10000.0, exact: bool = True):
    """RMSNorm over each token's H*D channels, then 3D RoPE in each head (bsa_oracle.c).

    x: uint16 [B, S, H, D] bf16 bits, token-major (a projection's output viewed per head);
    w: uint16 [H*D] bf16 bits; grid: (Gt, Gh, Gw) with Gt*Gh*Gw = S.
    Returns (y fp64 [B, H, S, D], y16 uint16 [B, H, S, D]: y rounded to bf16); y is None
    when exact is False (large inputs)."""
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w).reshape(-1)
    if x.dtype != np.uint16 or x.ndim != 4 or w.dtype != np.uint16:
        raise ValueError("expected x uint16 [B, S, H, D] and w uint16 [H*D]")
    B, S, H, D = x.shape
    gt, gh, gw = (int(g) for g in grid)
    if gt * gh * gw != S or w.size != H * D:
        raise ValueError("grid product must equal S and w must hold H*D values")
    y = np.empty((B, H, S, D), dtype=np.float64) if exact else None
    y16 = np.empty((B, H, S, D), dtype=np.uint16)
    _load().oracle_norm_rope(_ptr(x), _ptr(w), B, S, H, D, gt, gh, gw, float(eps), float(theta), _ptr(y), _ptr(y16))
    return y, y16
