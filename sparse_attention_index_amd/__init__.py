"""Python binding of libdsa.so, the MI355X (gfx950) DeepSeek Sparse
Attention hot-path library declared in include/dsa.h.

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch provides device memory and the current HIP stream. The library
must be built (``python -m sparse_attention_index_amd.build``); there is
no fallback path.

Calls (same names as the C ABI, without the ``dsa_`` prefix):
    rope_table(P, yarn=..., ...)            -> (cos, sin) float32 [P, 32]
    indexer(q_raw, w, pos, cos, sin, k_cache, k_scale, k_raw=None, ...)
                                            -> scores float32 [B, S, Lmax]
    topk(scores, pos, K)                    -> idx int32 [B, S, K]
    sparse_mla(q, latent, rope, idx, scale) -> out bf16 [B, S, Hq, 512] (, lse)
    sparse_mla_noalloc(q, latent, rope, idx, scale, out, lse=None)
                                            (no workspace, nothing allocated)
    mla_append(latent_new, kpe_new, pos, cos, sin, latent, rope, q=None)
    mla_kv_up(latent, wkv_b)                -> kv bf16 [B, L, Hq, 256]
    mla_absorb_q(q_nope, wkv_b)             -> bf16 [B, S, Hq, 512]
    mla_absorb_o(x, wkv_b)                  -> bf16 [B, S, Hq, 128]
    sparse_mha(q, kv, rope, idx, scale, pos=None)
                                            -> out bf16 [B, S, Hq, 128]
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_OK = 0
DSA_ERR_SCRATCH = 7
MLA_NOALLOC_MAX_BYTES = 56 << 20
DSA_DTYPE_F32 = 0
DSA_DTYPE_BF16 = 1
INDEX_DIM = 128
LATENT_DIM = 512
ROPE_DIM = 64
MAX_TOPK = 2048
APPEND_ONLY = 1
HADAMARD = 2
POW2_SCALE = 4

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_sz = ctypes.c_size_t


class RopeTableArgs(ctypes.Structure):
    _fields_ = [("P", _i32), ("yarn", _i32), ("orig_len", _i32), ("theta", _f32),
                ("factor", _f32), ("beta_fast", _f32), ("beta_slow", _f32),
                ("cos_out", _vp), ("sin_out", _vp)]


class IndexerArgs(ctypes.Structure):
    _fields_ = [("B", _i32), ("S", _i32), ("H", _i32), ("Lmax", _i32), ("P", _i32),
                ("act_dtype", _i32), ("q_raw", _vp), ("k_raw", _vp), ("pos", _vp),
                ("rope_cos", _vp), ("rope_sin", _vp), ("w", _vp), ("k_cache", _vp),
                ("k_scale", _vp), ("q_fp8", _vp), ("q_scale", _vp), ("scores", _vp),
                ("ld_scores", _i64), ("flags", ctypes.c_uint32), ("workspace", _vp),
                ("workspace_bytes", _sz), ("block_table", _vp), ("page_size", _i32), ("max_pages", _i32), ("num_pages", _i32)]


class TopkArgs(ctypes.Structure):
    _fields_ = [("B", _i32), ("S", _i32), ("Lmax", _i32), ("K", _i32), ("scores", _vp),
                ("ld_scores", _i64), ("pos", _vp), ("idx", _vp), ("count", _vp),
                ("workspace", _vp), ("workspace_bytes", _sz)]


class MlaArgs(ctypes.Structure):
    _fields_ = [("B", _i32), ("S", _i32), ("Hq", _i32), ("Lmax", _i32), ("K", _i32),
                ("q", _vp), ("latent", _vp), ("latent_row_stride", _i64),
                ("latent_batch_stride", _i64), ("rope", _vp), ("rope_row_stride", _i64),
                ("rope_batch_stride", _i64), ("idx", _vp), ("scale", _f32), ("out", _vp),
                ("lse", _vp), ("workspace", _vp), ("workspace_bytes", _sz),
                ("block_table", _vp), ("page_size", _i32), ("max_pages", _i32), ("num_pages", _i32)]


class MlaAppendArgs(ctypes.Structure):
    _fields_ = [("B", _i32), ("S", _i32), ("Hq", _i32), ("Lmax", _i32), ("P", _i32),
                ("latent_new", _vp), ("kpe_new", _vp), ("pos", _vp), ("rope_cos", _vp),
                ("rope_sin", _vp), ("latent", _vp), ("latent_row_stride", _i64),
                ("latent_batch_stride", _i64), ("rope", _vp), ("rope_row_stride", _i64),
                ("rope_batch_stride", _i64), ("q", _vp),
                ("block_table", _vp), ("page_size", _i32), ("max_pages", _i32), ("num_pages", _i32)]


class MlaProjArgs(ctypes.Structure):
    _fields_ = [("B", _i32), ("rows", _i32), ("Hq", _i32), ("wkv_b", _vp), ("x", _vp),
                ("x_row_stride", _i64), ("x_batch_stride", _i64), ("x_head_stride", _i64),
                ("y", _vp), ("y_row_stride", _i64), ("y_batch_stride", _i64),
                ("y_head_stride", _i64)]


class MhaArgs(ctypes.Structure):
    _fields_ = [("B", _i32), ("S", _i32), ("Hq", _i32), ("Lmax", _i32), ("K", _i32),
                ("q", _vp), ("kv", _vp), ("rope", _vp), ("rope_row_stride", _i64),
                ("rope_batch_stride", _i64), ("idx", _vp), ("pos", _vp), ("scale", _f32),
                ("out", _vp), ("workspace", _vp), ("workspace_bytes", _sz)]


EXPORTS = ("dsa_rope_table", "dsa_indexer_workspace", "dsa_indexer", "dsa_topk_workspace",
           "dsa_topk", "dsa_sparse_mla_workspace", "dsa_sparse_mla", "dsa_mla_append",
           "dsa_mla_kv_up", "dsa_mla_absorb_q", "dsa_mla_absorb_o", "dsa_sparse_mha_workspace",
           "dsa_sparse_mha", "dsa_sparse_mla_noalloc", "dsa_status_str", "dsa_abi_version")

_lib = None


class DSAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


def lib():
    """Load libdsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m sparse_attention_index_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.dsa_status_str.restype = ctypes.c_char_p
    L.dsa_status_str.argtypes = [ctypes.c_int]
    L.dsa_abi_version.restype = ctypes.c_int
    L.dsa_abi_version.argtypes = []
    for name, st in (("rope_table", RopeTableArgs), ("indexer", IndexerArgs),
                     ("topk", TopkArgs), ("sparse_mla", MlaArgs),
                     ("mla_append", MlaAppendArgs), ("mla_kv_up", MlaProjArgs),
                     ("mla_absorb_q", MlaProjArgs), ("mla_absorb_o", MlaProjArgs),
                     ("sparse_mha", MhaArgs)):
        fn = getattr(L, "dsa_" + name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.POINTER(st), _vp]
        if name in ("indexer", "topk", "sparse_mla", "sparse_mha"):
            ws = getattr(L, f"dsa_{name}_workspace")
            ws.restype = ctypes.c_int
            ws.argtypes = [ctypes.POINTER(st), ctypes.POINTER(_sz)]
    L.dsa_sparse_mla_noalloc.restype = ctypes.c_int
    L.dsa_sparse_mla_noalloc.argtypes = [ctypes.POINTER(MlaArgs), _vp]
    _lib = L
    return L


def _check(code: int):
    if code != DSA_OK:
        raise DSAError(code, lib().dsa_status_str(code).decode())


def status_str(code: int) -> str:
    return lib().dsa_status_str(code).decode()


def _stream():
    import torch
    return _vp(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else _vp(t.data_ptr())


def _need(t, name, dtype, shape=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


# ---------------------------------------------------------------- calls --

def rope_table(P: int, yarn: bool = False, theta: float = 10000.0, orig_len: int = 4096,
               factor: float = 40.0, beta_fast: float = 32.0, beta_slow: float = 1.0,
               device="cuda"):
    import torch
    cos = torch.empty((P, ROPE_DIM // 2), dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    a = RopeTableArgs(P, int(bool(yarn)), orig_len, theta, factor, beta_fast, beta_slow,
                      _ptr(cos), _ptr(sin))
    _check(lib().dsa_rope_table(ctypes.byref(a), _stream()))
    return cos, sin


class Paging:
    """A paged cache layout: block_table int32 [B, max_pages] (device) maps
    page p // page_size of batch row b to a page of a pool of num_pages
    pages; the caches passed with it are pools [num_pages, page_size, ...]."""

    def __init__(self, block_table, page_size: int, num_pages: int):
        import torch
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or \
                not block_table.is_contiguous() or not block_table.is_cuda:
            raise ValueError("block_table must be a contiguous int32 device tensor [B, max_pages]")
        self.block_table, self.page_size, self.num_pages = block_table, int(page_size), int(num_pages)
        self.max_pages = block_table.shape[1]

    @property
    def lmax(self) -> int:
        return self.max_pages * self.page_size

    def set_fields(self, a):
        a.block_table = _ptr(self.block_table)
        a.page_size, a.max_pages, a.num_pages = self.page_size, self.max_pages, self.num_pages


def _cache_rows(t, paging, B):
    """(Lmax, leading shape) of a dense [B, Lmax, ...] cache or a pool."""
    if paging is None:
        return t.shape[1], (B, t.shape[1])
    return paging.lmax, (paging.num_pages, paging.page_size)


def _prep_flags(hadamard, pow2_scale):
    return (HADAMARD if hadamard else 0) | (POW2_SCALE if pow2_scale else 0)


def indexer_args(q_raw, w, pos, cos, sin, k_cache, k_scale, scores, k_raw=None, q_fp8=None,
                 q_scale=None, workspace=None, hadamard=False, pow2_scale=False,
                 paging=None) -> IndexerArgs:
    import torch
    B, S, H, D = q_raw.shape
    Lmax, lead = _cache_rows(k_cache, paging, B)
    dt = {torch.float32: DSA_DTYPE_F32, torch.bfloat16: DSA_DTYPE_BF16}.get(q_raw.dtype)
    if dt is None:
        raise TypeError("q_raw must be float32 or bfloat16")
    _need(q_raw, "q_raw", q_raw.dtype, (B, S, H, INDEX_DIM))
    _need(w, "w", torch.float32, (B, S, H))
    _need(pos, "pos", torch.int32, (B, S))
    _need(cos, "cos", torch.float32)
    _need(sin, "sin", torch.float32, cos.shape)
    _need(k_cache, "k_cache", torch.uint8, lead + (INDEX_DIM,))
    _need(k_scale, "k_scale", torch.float32, lead)
    if scores.dim() != 3 or scores.shape[:2] != (B, S) or scores.stride(2) != 1 \
            or scores.stride(0) != S * scores.stride(1):
        raise ValueError("scores must be [B, S, >=Lmax] with unit inner stride")
    if not scores.is_cuda or scores.dtype != torch.float32:
        raise TypeError("scores must be a float32 device tensor")
    if k_raw is not None:
        _need(k_raw, "k_raw", q_raw.dtype, (B, S, INDEX_DIM))
    if q_fp8 is not None:
        _need(q_fp8, "q_fp8", torch.uint8, (B, S, H, INDEX_DIM))
        _need(q_scale, "q_scale", torch.float32, (B, S, H))
    a = IndexerArgs(B, S, H, Lmax, cos.shape[0], dt, _ptr(q_raw), _ptr(k_raw), _ptr(pos),
                    _ptr(cos), _ptr(sin), _ptr(w), _ptr(k_cache), _ptr(k_scale),
                    _ptr(q_fp8), _ptr(q_scale), _ptr(scores), scores.stride(1),
                    _prep_flags(hadamard, pow2_scale), _ptr(workspace),
                    0 if workspace is None else workspace.numel())
    if paging is not None:
        paging.set_fields(a)
    return a


def indexer_append(k_raw, pos, cos, sin, k_cache, k_scale, hadamard=False, pow2_scale=False,
                   paging=None):
    """Call 1 with DSA_INDEXER_APPEND_ONLY: rotate, quantise and write the
    key rows k_raw [B, S, 128] into k_cache/k_scale at pos [B, S]."""
    import torch
    B, S = pos.shape
    Lmax, lead = _cache_rows(k_cache, paging, B)
    dt = {torch.float32: DSA_DTYPE_F32, torch.bfloat16: DSA_DTYPE_BF16}.get(k_raw.dtype)
    if dt is None:
        raise TypeError("k_raw must be float32 or bfloat16")
    _need(k_raw, "k_raw", k_raw.dtype, (B, S, INDEX_DIM))
    _need(pos, "pos", torch.int32, (B, S))
    _need(cos, "cos", torch.float32)
    _need(sin, "sin", torch.float32, cos.shape)
    _need(k_cache, "k_cache", torch.uint8, lead + (INDEX_DIM,))
    _need(k_scale, "k_scale", torch.float32, lead)
    a = IndexerArgs(B, S, 1, Lmax, cos.shape[0], dt, None, _ptr(k_raw), _ptr(pos), _ptr(cos),
                    _ptr(sin), None, _ptr(k_cache), _ptr(k_scale), None, None, None, Lmax,
                    APPEND_ONLY | _prep_flags(hadamard, pow2_scale), None, 0)
    if paging is not None:
        paging.set_fields(a)
    _check(lib().dsa_indexer(ctypes.byref(a), _stream()))


def indexer_workspace_bytes(args: IndexerArgs) -> int:
    n = _sz(0)
    _check(lib().dsa_indexer_workspace(ctypes.byref(args), ctypes.byref(n)))
    return n.value


def _workspace(nbytes, device):
    import torch
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def indexer(q_raw, w, pos, cos, sin, k_cache, k_scale, scores=None, k_raw=None, q_fp8=None,
            q_scale=None, workspace=None, hadamard=False, pow2_scale=False, paging=None):
    """Call 1: append k_raw rows (if given) and score every causal key.
    Returns scores [B, S, Lmax] float32 (entries past each row's position
    are left as they were)."""
    import torch
    B, S = q_raw.shape[:2]
    if scores is None:
        L = k_cache.shape[1] if paging is None else paging.lmax
        scores = torch.empty((B, S, L), dtype=torch.float32, device=q_raw.device)
    a = indexer_args(q_raw, w, pos, cos, sin, k_cache, k_scale, scores, k_raw, q_fp8, q_scale,
                     workspace, hadamard, pow2_scale, paging)
    need = indexer_workspace_bytes(a)
    if need and (workspace is None or workspace.numel() < need):
        workspace = _workspace(need, q_raw.device)
        a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    _check(lib().dsa_indexer(ctypes.byref(a), _stream()))
    return scores


def topk_args(scores, pos, K, idx, count=None, workspace=None) -> TopkArgs:
    import torch
    B, S = pos.shape
    _need(pos, "pos", torch.int32, (B, S))
    _need(idx, "idx", torch.int32, (B, S, K))
    if count is not None:
        _need(count, "count", torch.int32, (B, S))
    if scores.dim() != 3 or scores.shape[:2] != (B, S) or scores.stride(2) != 1 \
            or scores.stride(0) != S * scores.stride(1) or scores.dtype != torch.float32:
        raise ValueError("scores must be float32 [B, S, L] with unit inner stride")
    return TopkArgs(B, S, scores.shape[2], K, _ptr(scores), scores.stride(1), _ptr(pos),
                    _ptr(idx), _ptr(count), _ptr(workspace),
                    0 if workspace is None else workspace.numel())


def topk_workspace_bytes(args: TopkArgs) -> int:
    n = _sz(0)
    _check(lib().dsa_topk_workspace(ctypes.byref(args), ctypes.byref(n)))
    return n.value


def topk_workspace(scores, pos, K: int):
    """A workspace for topk() on these shapes (reusable across calls on one
    stream; its contents between calls do not matter)."""
    import torch
    B, S = pos.shape
    idx = torch.empty((B, S, K), dtype=torch.int32, device=scores.device)
    n = topk_workspace_bytes(topk_args(scores, pos, K, idx))
    return torch.empty(max(n, 1), dtype=torch.uint8, device=scores.device)


def topk(scores, pos, K: int, idx=None, count=None, workspace=None):
    """Call 2: causal top-K of every score row; returns idx [B, S, K] int32.
    `workspace` (from topk_workspace()) is allocated per call when omitted."""
    import torch
    B, S = pos.shape
    if idx is None:
        idx = torch.empty((B, S, K), dtype=torch.int32, device=scores.device)
    a = topk_args(scores, pos, K, idx, count, workspace)
    need = topk_workspace_bytes(a)
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
        a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    _check(lib().dsa_topk(ctypes.byref(a), _stream()))
    return idx


def _check_latent_caches(latent, rope, paging, B):
    import torch
    for name, t, d in (("latent", latent, LATENT_DIM), ("rope", rope, ROPE_DIM)):
        lead = B if paging is None else paging.num_pages
        if t.dtype != torch.bfloat16 or not t.is_cuda or t.dim() != 3 or t.shape[0] != lead \
                or t.shape[2] != d or t.stride(2) != 1:
            raise ValueError(f"{name} must be a bf16 device tensor [{'B, Lmax' if paging is None else 'num_pages, page_size'}, {d}] "
                             "with unit inner stride")
        if paging is not None and t.shape[1] != paging.page_size:
            raise ValueError(f"{name} pool pages must hold page_size rows")
    if latent.shape[1] != rope.shape[1]:
        raise ValueError("latent and rope must have the same number of rows")
    return latent.shape[1] if paging is None else paging.lmax


def mla_args(q, latent, rope, idx, scale, out, lse=None, workspace=None, paging=None) -> MlaArgs:
    import torch
    B, S, Hq, Dq = q.shape
    K = idx.shape[-1]
    _need(q, "q", torch.bfloat16, (B, S, Hq, LATENT_DIM + ROPE_DIM))
    _need(idx, "idx", torch.int32, (B, S, K))
    _need(out, "out", torch.bfloat16, (B, S, Hq, LATENT_DIM))
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, S, Hq))
    Lmax = _check_latent_caches(latent, rope, paging, B)
    a = MlaArgs(B, S, Hq, Lmax, K, _ptr(q), _ptr(latent), latent.stride(1),
                latent.stride(0), _ptr(rope), rope.stride(1), rope.stride(0), _ptr(idx),
                float(scale), _ptr(out), _ptr(lse), _ptr(workspace),
                0 if workspace is None else workspace.numel())
    if paging is not None:
        paging.set_fields(a)
    return a


def sparse_mla_workspace_bytes(args: MlaArgs) -> int:
    n = _sz(0)
    _check(lib().dsa_sparse_mla_workspace(ctypes.byref(args), ctypes.byref(n)))
    return n.value


def sparse_mla(q, latent, rope, idx, scale: float, out=None, lse=None, workspace=None,
               return_lse: bool = False, paging=None):
    """Call 3: absorbed sparse MLA; returns out [B, S, Hq, 512] bf16 (and lse)."""
    import torch
    B, S, Hq, _ = q.shape
    if out is None:
        out = torch.empty((B, S, Hq, LATENT_DIM), dtype=torch.bfloat16, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((B, S, Hq), dtype=torch.float32, device=q.device)
    a = mla_args(q, latent, rope, idx, scale, out, lse, workspace, paging)
    need = sparse_mla_workspace_bytes(a)
    if need and (workspace is None or workspace.numel() < need):
        workspace = _workspace(need, q.device)
        a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    _check(lib().dsa_sparse_mla(ctypes.byref(a), _stream()))
    return (out, lse) if return_lse else out


def sparse_mla_noalloc(q, latent, rope, idx, scale: float, out, lse=None, paging=None):
    """Call 3 through dsa_sparse_mla_noalloc: the caller passes the outputs
    (out [B, S, Hq, 512] bf16, optional lse [B, S, Hq] float32); the key-split
    partials go to the library's static scratch, nothing is allocated."""
    a = mla_args(q, latent, rope, idx, scale, out, lse, None, paging)
    _check(lib().dsa_sparse_mla_noalloc(ctypes.byref(a), _stream()))
    return out


def mla_append(latent_new, kpe_new, pos, cos, sin, latent, rope, q=None, paging=None):
    """Write latent_new [B, S, 512] and the interleaved-RoPE-rotated kpe_new
    [B, S, 64] into the caches latent / rope ([B, Lmax, 512] / [B, Lmax, 64]
    views with unit inner stride) at pos [B, S]; if q [B, S, Hq, 576] is
    given, its rope part is rotated in place."""
    import torch
    B, S = pos.shape
    _need(pos, "pos", torch.int32, (B, S))
    _need(latent_new, "latent_new", torch.bfloat16, (B, S, LATENT_DIM))
    _need(kpe_new, "kpe_new", torch.bfloat16, (B, S, ROPE_DIM))
    _need(cos, "cos", torch.float32)
    _need(sin, "sin", torch.float32, cos.shape)
    Lmax = _check_latent_caches(latent, rope, paging, B)
    Hq = 0
    if q is not None:
        Hq = q.shape[2]
        _need(q, "q", torch.bfloat16, (B, S, Hq, LATENT_DIM + ROPE_DIM))
    a = MlaAppendArgs(B, S, Hq, Lmax, cos.shape[0], _ptr(latent_new), _ptr(kpe_new),
                      _ptr(pos), _ptr(cos), _ptr(sin), _ptr(latent), latent.stride(1),
                      latent.stride(0), _ptr(rope), rope.stride(1), rope.stride(0), _ptr(q))
    if paging is not None:
        paging.set_fields(a)
    _check(lib().dsa_mla_append(ctypes.byref(a), _stream()))


# ------------------------------------------------------------ projections --

def _proj_view(t, name, width, heads=None):
    """(row stride, batch stride, head stride) of a bf16 device tensor
    [B, rows, width] or [B, rows, Hq, width] with unit inner stride."""
    import torch
    dims = 3 if heads is None else 4
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.bfloat16 \
            or t.dim() != dims or t.shape[-1] != width or t.stride(-1) != 1 \
            or (heads is not None and t.shape[2] != heads):
        shape = "[B, rows, %d]" % width if heads is None else "[B, rows, Hq, %d]" % width
        raise ValueError(f"{name} must be a bf16 device tensor {shape} with unit inner stride")
    return t.stride(1), t.stride(0), (0 if heads is None else t.stride(2))


def _wkv_b(wkv_b):
    import torch
    _need(wkv_b, "wkv_b", torch.bfloat16)
    if wkv_b.dim() != 3 or tuple(wkv_b.shape[1:]) != (256, LATENT_DIM):
        raise ValueError("wkv_b must be [Hq, 256, 512] (W_UK rows 0..127, W_UV rows 128..255)")
    return wkv_b.shape[0]


def mla_kv_up(latent, wkv_b, out=None):
    """Up-projection of the multi-head prefill form: latent [B, L, 512] ->
    kv [B, L, Hq, 256] (k_nope then v per head)."""
    import torch
    Hq = _wkv_b(wkv_b)
    B, L = latent.shape[:2]
    xs = _proj_view(latent, "latent", LATENT_DIM)
    if out is None:
        out = torch.empty((B, L, Hq, 256), dtype=torch.bfloat16, device=latent.device)
    ys = _proj_view(out, "out", 256, Hq)
    if tuple(out.shape[:2]) != (B, L) or out.stride(2) != 256:
        raise ValueError("out must be [B, L, Hq, 256] with contiguous heads")
    a = MlaProjArgs(B, L, Hq, _ptr(wkv_b), _ptr(latent), xs[0], xs[1], 0, _ptr(out), ys[0],
                    ys[1], 0)
    _check(lib().dsa_mla_kv_up(ctypes.byref(a), _stream()))
    return out


def _absorb(fn, x, wkv_b, out, din, dout):
    import torch
    Hq = _wkv_b(wkv_b)
    xs = _proj_view(x, "x", din, Hq)
    B, S = x.shape[:2]
    if out is None:
        out = torch.empty((B, S, Hq, dout), dtype=torch.bfloat16, device=x.device)
    ys = _proj_view(out, "out", dout, Hq)
    if tuple(out.shape[:2]) != (B, S):
        raise ValueError("out must match x's leading dimensions")
    a = MlaProjArgs(B, S, Hq, _ptr(wkv_b), _ptr(x), xs[0], xs[1], xs[2], _ptr(out), ys[0],
                    ys[1], ys[2])
    _check(fn(ctypes.byref(a), _stream()))
    return out


def mla_absorb_q(q_nope, wkv_b, out=None):
    """q_nope [B, S, Hq, 128] -> q_nope . W_UK [B, S, Hq, 512]; out may be a
    view such as q[..., :512] of a [B, S, Hq, 576] query."""
    return _absorb(lib().dsa_mla_absorb_q, q_nope, wkv_b, out, 128, LATENT_DIM)


def mla_absorb_o(x, wkv_b, out=None):
    """x [B, S, Hq, 512] (latent attention output) -> x . W_UV^T [B, S, Hq, 128]."""
    return _absorb(lib().dsa_mla_absorb_o, x, wkv_b, out, LATENT_DIM, 128)


def mha_args(q, kv, rope, idx, scale, out, pos=None, workspace=None) -> MhaArgs:
    import torch
    B, S, Hq, _ = q.shape
    K = idx.shape[-1]
    _need(q, "q", torch.bfloat16, (B, S, Hq, 192))
    _need(kv, "kv", torch.bfloat16)
    if kv.dim() != 4 or kv.shape[0] != B or kv.shape[2] != Hq or kv.shape[3] != 256:
        raise ValueError("kv must be [B, Lmax, Hq, 256]")
    Lmax = kv.shape[1]
    if rope.dtype != torch.bfloat16 or not rope.is_cuda or rope.dim() != 3 or \
            rope.shape[0] != B or rope.shape[1] != Lmax or rope.shape[2] != ROPE_DIM or \
            rope.stride(2) != 1:
        raise ValueError("rope must be a bf16 device tensor [B, Lmax, 64] with unit inner stride")
    _need(idx, "idx", torch.int32, (B, S, K))
    _need(out, "out", torch.bfloat16, (B, S, Hq, 128))
    if pos is not None:
        _need(pos, "pos", torch.int32, (B, S))
    return MhaArgs(B, S, Hq, Lmax, K, _ptr(q), _ptr(kv), _ptr(rope), rope.stride(1),
                   rope.stride(0), _ptr(idx), _ptr(pos), float(scale), _ptr(out),
                   _ptr(workspace), 0 if workspace is None else workspace.numel())


def sparse_mha_tiles_offset(B: int, S: int, Lmax: int) -> int:
    """Byte offset of the key-tile lists inside the workspace: after the bit
    masks ([B*S][2*ceil(Lmax/64)] words), rounded up to 256. The lists are
    [B*ceil(S/128)][ceil(Lmax/64) + 1] int4: entry 0 holds the count, then
    (tile, union bits low, union bits high, 0); 256 zero bytes follow them
    (at the next multiple of 256)."""
    nkt = (Lmax + 63) // 64
    return (B * S * 2 * nkt * 4 + 255) // 256 * 256


def sparse_mha_workspace_bytes(args: MhaArgs) -> int:
    n = _sz(0)
    _check(lib().dsa_sparse_mha_workspace(ctypes.byref(args), ctypes.byref(n)))
    return n.value


def sparse_mha(q, kv, rope, idx, scale: float, pos=None, out=None, workspace=None):
    """Multi-head (non-absorbed) sparse prefill attention: q [B, S, Hq, 192],
    kv [B, Lmax, Hq, 256] (mla_kv_up), rope [B, Lmax, 64], idx [B, S, K],
    optional pos [B, S] (causal mask) -> out bf16 [B, S, Hq, 128]."""
    import torch
    B, S, Hq, _ = q.shape
    if out is None:
        out = torch.empty((B, S, Hq, 128), dtype=torch.bfloat16, device=q.device)
    a = mha_args(q, kv, rope, idx, scale, out, pos, workspace)
    need = sparse_mha_workspace_bytes(a)
    if workspace is None or workspace.numel() < need:
        workspace = _workspace(need, q.device)
        a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    _check(lib().dsa_sparse_mha(ctypes.byref(a), _stream()))
    return out
