"""CPU oracle for the DeepSeek Sparse Attention hot path (numpy front end).

TEST INFRASTRUCTURE, NOT PRODUCT CODE. This package is the plain reference
the GPU library is checked against. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it. It shares no code with the GPU
library and the GPU library never imports it.

All arithmetic lives in oracle.c (plain C loops, double accumulation); this
module only marshals numpy arrays. bfloat16 data travels as uint16 bit
patterns; `bf16_bits_to_f32` widens them exactly.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_i32 = ctypes.c_int
_f64 = ctypes.c_double
_ptr = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sigs = {
        "orc_e4m3_decode": (_f64, [ctypes.c_uint8]),
        "orc_e4m3_encode": (ctypes.c_uint8, [ctypes.c_float]),
        "orc_e4m3_encode_array": (None, [_i64, _ptr, _ptr]),
        "orc_e4m3_decode_array": (None, [_i64, _ptr, _ptr]),
        "orc_round_bf16": (ctypes.c_float, [ctypes.c_float]),
        "orc_round_bf16_array": (None, [_i64, _ptr, _ptr]),
        "orc_rope_table": (None, [_i32, _i32, _f64, _i32, _i32, _f64, _f64, _f64, _ptr, _ptr]),
        "orc_rope_freqs": (None, [_i32, _f64, _i32, _i32, _f64, _f64, _f64, _ptr]),
        "orc_rope_rows": (None, [_i64, _i32, _i32, _i32, _ptr, _ptr, _ptr, _ptr, _i32, _ptr]),
        "orc_quantize_rows": (None, [_i64, _ptr, _ptr, _ptr]),
        "orc_quantize_rows_pow2": (None, [_i64, _ptr, _ptr, _ptr]),
        "orc_hadamard_rows": (None, [_i64, _ptr, _i32, _ptr]),
        "orc_dequantize_rows": (None, [_i64, _ptr, _ptr, _ptr]),
        "orc_indexer_scores": (None, [_i32, _i32, _i32, _i32, _i32, _ptr, _ptr, _ptr, _ptr, _ptr]),
        "orc_topk": (None, [_i64, _i64, _ptr, _ptr, _i32, _ptr]),
        "orc_sparse_mla": (None, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _ptr, _ptr, _ptr,
                                  _ptr, _f64, _ptr, _ptr]),
        "orc_mla_mha": (None, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _ptr, _ptr,
                               _ptr, _ptr, _ptr, _ptr, _f64, _ptr]),
        "orc_sparse_mha": (None, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _ptr, _ptr,
                                  _ptr, _ptr, _ptr, _f64, _ptr]),
        "orc_num_threads": (_i32, []),
        "orc_set_num_threads": (None, [_i32]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return _load().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Threads the following oracle calls use (OpenMP)."""
    _load().orc_set_num_threads(int(n))


# ---------------------------------------------------------------- dtypes --

def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def e4m3_decode(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().orc_e4m3_decode_array(c.size, _p(c), _p(out))
    return out


def e4m3_encode(x) -> np.ndarray:
    a = _c(x, np.float32)
    out = np.empty(a.shape, np.uint8)
    _load().orc_e4m3_encode_array(a.size, _p(a), _p(out))
    return out


def round_bf16(x) -> np.ndarray:
    a = _c(x, np.float32)
    out = np.empty(a.shape, np.float32)
    _load().orc_round_bf16_array(a.size, _p(a), _p(out))
    return out


# ------------------------------------------------------------------ rope --

def rope_freqs(rope_dim=64, theta=10000.0, yarn=False, orig_len=4096, factor=40.0,
               beta_fast=32.0, beta_slow=1.0) -> np.ndarray:
    assert rope_dim % 2 == 0 and rope_dim <= 512
    out = np.empty(rope_dim // 2, np.float32)
    _load().orc_rope_freqs(rope_dim, theta, int(bool(yarn)), orig_len, factor, beta_fast,
                           beta_slow, _p(out))
    return out


def rope_table(P, rope_dim=64, theta=10000.0, yarn=False, orig_len=4096, factor=40.0,
               beta_fast=32.0, beta_slow=1.0):
    """(cos, sin), each float32 [P, rope_dim/2]."""
    assert rope_dim % 2 == 0 and rope_dim <= 512
    cos = np.empty((P, rope_dim // 2), np.float32)
    sin = np.empty((P, rope_dim // 2), np.float32)
    _load().orc_rope_table(P, rope_dim, theta, int(bool(yarn)), orig_len, factor, beta_fast,
                           beta_slow, _p(cos), _p(sin))
    return cos, sin


def rope(x, pos, cos, sin, rope_dim=64, interleaved=False, out_bf16=False) -> np.ndarray:
    """Rotate the first rope_dim features of each row of x (float32 [..., W])."""
    a = _c(x, np.float32)
    width = a.shape[-1]
    nrows = a.size // width
    p = _c(np.broadcast_to(pos, a.shape[:-1]), np.int32)
    c = _c(cos, np.float32)
    s = _c(sin, np.float32)
    assert p.size == nrows and p.max(initial=0) < c.shape[0] and p.min(initial=0) >= 0
    out = np.empty_like(a)
    _load().orc_rope_rows(nrows, width, rope_dim, int(bool(interleaved)), _p(a), _p(p), _p(c),
                          _p(s), int(bool(out_bf16)), _p(out))
    return out


# ------------------------------------------------------------ quantiser --

def quantize(x, pow2=False):
    """Block FP8: x float32 [..., 128] -> (codes uint8 [..., 128], scales float32 [...]).
    pow2: scales rounded up to a power of two."""
    a = _c(x, np.float32)
    assert a.shape[-1] == 128
    nrows = a.size // 128
    codes = np.empty(a.shape, np.uint8)
    scales = np.empty(a.shape[:-1], np.float32)
    fn = _load().orc_quantize_rows_pow2 if pow2 else _load().orc_quantize_rows
    fn(nrows, _p(a), _p(codes), _p(scales))
    return codes, scales


def hadamard(x, out_bf16=False) -> np.ndarray:
    """y = H_128 x / sqrt(128) per row of x float32 [..., 128] (float32 FWHT)."""
    a = _c(x, np.float32)
    assert a.shape[-1] == 128
    out = np.empty_like(a)
    _load().orc_hadamard_rows(a.size // 128, _p(a), int(bool(out_bf16)), _p(out))
    return out


def dequantize(codes, scales) -> np.ndarray:
    c = _c(codes, np.uint8)
    s = _c(scales, np.float32)
    assert c.shape[-1] == 128 and s.size == c.size // 128
    out = np.empty(c.shape, np.float64)
    _load().orc_dequantize_rows(s.size, _p(c), _p(s), _p(out))
    return out


def indexer_prepare(x, pos, cos, sin, bf16_input: bool, hadamard_rot=False, pow2=False):
    """Indexer q or k rows as the pages prepare them: non-interleaved RoPE on
    features 0..63 in float32, cast back to the input dtype, optionally the
    Hadamard rotation (also cast back), block FP8 (optionally with
    power-of-two scales).

    x: float32 [..., 128] holding the input values (bf16 values when
    bf16_input); pos broadcastable to x.shape[:-1].
    Returns (codes, scales, rotated float32)."""
    rot = rope(x, pos, cos, sin, rope_dim=64, interleaved=False, out_bf16=bf16_input)
    if hadamard_rot:
        rot = hadamard(rot, out_bf16=bf16_input)
    codes, scales = quantize(rot, pow2=pow2)
    return codes, scales, rot


# --------------------------------------------------------------- indexer --

def indexer_scores(q, w, k, n_valid) -> np.ndarray:
    """q [B,S,H,D], w [B,S,H], k [B,Lmax,D] (real values), n_valid [B,S].
    Returns float64 [B,S,Lmax]; entries at s >= n_valid are NaN."""
    qq = _c(q, np.float64)
    ww = _c(w, np.float64)
    kk = _c(k, np.float64)
    nv = _c(n_valid, np.int32)
    B, S, H, D = qq.shape
    Lmax = kk.shape[1]
    assert kk.shape == (B, Lmax, D) and ww.shape == (B, S, H) and nv.shape == (B, S)
    assert nv.min(initial=1) >= 0 and nv.max(initial=0) <= Lmax
    out = np.full((B, S, Lmax), np.nan, np.float64)
    _load().orc_indexer_scores(B, S, H, D, Lmax, _p(qq), _p(ww), _p(kk), _p(nv), _p(out))
    return out


# ------------------------------------------------------------------ topk --

def topk(scores, n_valid, K) -> np.ndarray:
    """scores [..., L] (float), n_valid [...] -> int32 [..., K] ascending, -1 padded."""
    sc = _c(scores, np.float64)
    L = sc.shape[-1]
    nrows = sc.size // L if L else int(np.prod(sc.shape[:-1]))
    nv = _c(np.broadcast_to(n_valid, sc.shape[:-1]), np.int32)
    assert nv.size == nrows and nv.max(initial=0) <= L and nv.min(initial=0) >= 0
    idx = np.empty(sc.shape[:-1] + (K,), np.int32)
    _load().orc_topk(nrows, L, _p(sc), _p(nv), K, _p(idx))
    return idx


# ------------------------------------------------------------------- mla --

def sparse_mla(q, latent, kpe, idx, scale):
    """q [B,S,Hq,Dl+Dr], latent [B,Lmax,Dl], kpe [B,Lmax,Dr], idx [B,S,K] int32.
    Returns (out float64 [B,S,Hq,Dl], lse float64 [B,S,Hq])."""
    qq = _c(q, np.float64)
    lat = _c(latent, np.float64)
    pe = _c(kpe, np.float64)
    ix = _c(idx, np.int32)
    B, S, Hq, Dq = qq.shape
    Lmax, Dl = lat.shape[1], lat.shape[2]
    Dr = pe.shape[2]
    K = ix.shape[-1]
    assert Dq == Dl + Dr and lat.shape[0] == B and pe.shape[:2] == (B, Lmax)
    assert ix.shape == (B, S, K) and ix.max(initial=-1) < Lmax
    out = np.empty((B, S, Hq, Dl), np.float64)
    lse = np.empty((B, S, Hq), np.float64)
    _load().orc_sparse_mla(B, S, Hq, Dl, Dr, Lmax, K, _p(qq), _p(lat), _p(pe), _p(ix),
                           float(scale), _p(out), _p(lse))
    return out, lse


def mla_mha(q_nope, q_pe, wkv_b, latent, kpe, idx, scale):
    """Non-absorbed form. q_nope [B,S,Hq,Dn], q_pe [B,S,Hq,Dr], wkv_b [Hq,Dn+Dv,Dl].
    Returns float64 [B,S,Hq,Dv]."""
    qn = _c(q_nope, np.float64)
    qp = _c(q_pe, np.float64)
    W = _c(wkv_b, np.float64)
    lat = _c(latent, np.float64)
    pe = _c(kpe, np.float64)
    ix = _c(idx, np.int32)
    B, S, Hq, Dn = qn.shape
    Dr = qp.shape[-1]
    Dl = lat.shape[2]
    Lmax = lat.shape[1]
    Dv = W.shape[1] - Dn
    K = ix.shape[-1]
    assert W.shape == (Hq, Dn + Dv, Dl) and ix.shape == (B, S, K)
    out = np.empty((B, S, Hq, Dv), np.float64)
    _load().orc_mla_mha(B, S, Hq, Dn, Dv, Dl, Dr, Lmax, K, _p(qn), _p(qp), _p(W), _p(lat),
                        _p(pe), _p(ix), float(scale), _p(out))
    return out


def sparse_mha(q, kv, kpe, idx, scale, pos=None, Dn=128):
    """Multi-head prefill attention over up-projected keys and values (page
    "RoPE coefficients", MLA prefill excerpt): q [B,S,Hq,Dn+Dr] (q_nope then
    q_pe), kv [B,Lmax,Hq,Dn+Dv] (k_nope then v), kpe [B,Lmax,Dr], idx [B,S,K];
    the selection is a set and, with pos [B,S], causally masked.
    Returns float64 [B,S,Hq,Dv]."""
    qq = _c(q, np.float64)
    kk = _c(kv, np.float64)
    pe = _c(kpe, np.float64)
    ix = _c(idx, np.int32)
    B, S, Hq, Dq = qq.shape
    Lmax, Dkv = kk.shape[1], kk.shape[3]
    Dr = pe.shape[2]
    Dv = Dkv - Dn
    K = ix.shape[-1]
    assert Dq == Dn + Dr and kk.shape[:3] == (B, Lmax, Hq) and pe.shape[:2] == (B, Lmax)
    assert ix.shape == (B, S, K)
    pp = None if pos is None else _c(np.broadcast_to(pos, (B, S)), np.int32)
    out = np.empty((B, S, Hq, Dv), np.float64)
    _load().orc_sparse_mha(B, S, Hq, Dn, Dv, Dr, Lmax, K, _p(qq), _p(kk), _p(pe), _p(ix),
                           None if pp is None else _p(pp), float(scale), _p(out))
    return out


# ----------------------------------------------------------- projections --
# wkv_b [Hq, Dn+Dv, Dl]: rows 0..Dn-1 of head h are W_UK (keys' non-rotary
# part), rows Dn.. are W_UV (values). Plain float64 matrix products.

def kv_up(latent, wkv_b):
    """Up-projection of the MLA prefill excerpt (page "RoPE coefficients"):
    kv = wkv_b(latent) viewed as [.., Hq, Dn+Dv]. latent [B,L,Dl] ->
    float64 [B,L,Hq,Dn+Dv]."""
    lat = _c(latent, np.float64)
    W = _c(wkv_b, np.float64)
    Hq, Dkv, Dl = W.shape
    B, L, _ = lat.shape
    y = lat.reshape(B * L, Dl) @ W.reshape(Hq * Dkv, Dl).T
    return y.reshape(B, L, Hq, Dkv)


def absorb_q(q_nope, wkv_b, Dn=128):
    """Query absorption of the MQA decode excerpt (page "Similarities"):
    q_lat[..., h, c] = sum_d q_nope[..., h, d] W_UK[h][d][c].
    q_nope [..., Hq, Dn] -> float64 [..., Hq, Dl]."""
    qn = _c(q_nope, np.float64)
    W = _c(wkv_b, np.float64)[:, :Dn]                     # [Hq, Dn, Dl]
    lead = qn.shape[:-2]
    Hq = qn.shape[-2]
    x = qn.reshape(-1, Hq, Dn).transpose(1, 0, 2)         # [Hq, R, Dn]
    y = np.matmul(x, W)                                   # [Hq, R, Dl]
    return y.transpose(1, 0, 2).reshape(lead + (Hq, W.shape[2]))


def absorb_o(x_lat, wkv_b, Dn=128):
    """Output absorption of the MQA decode excerpt (page "Similarities"):
    o[..., h, d] = sum_c x[..., h, c] W_UV[h][d][c].
    x_lat [..., Hq, Dl] -> float64 [..., Hq, Dv]."""
    xx = _c(x_lat, np.float64)
    W = _c(wkv_b, np.float64)[:, Dn:]                     # [Hq, Dv, Dl]
    lead = xx.shape[:-2]
    Hq, Dl = xx.shape[-2:]
    x = xx.reshape(-1, Hq, Dl).transpose(1, 0, 2)         # [Hq, R, Dl]
    y = np.matmul(x, W.transpose(0, 2, 1))                # [Hq, R, Dv]
    return y.transpose(1, 0, 2).reshape(lead + (Hq, W.shape[1]))


# ------------------------------------------------------------ whole path --

def decode_path(q_raw, k_cache_raw, pos, w, cos, sin, q_mla, latent, kpe, K, scale,
                bf16_input=True, quantized=True):
    """The whole hot path for one batch of query rows, in the pages' order:
    prepare q and k (RoPE + FP8), indexer score, causal top-k, sparse MLA.

    q_raw [B,S,H,128] float32 values, k_cache_raw [B,Lmax,128] float32 values
    (key s is rotated with position s), pos [B,S]; q_mla [B,S,Hq,Dl+Dr],
    latent [B,Lmax,Dl], kpe [B,Lmax,Dr] as float values.
    quantized=False skips the FP8 step (fp32 indexer, as the tiny config).
    Returns dict with scores, idx, out, lse and the FP8 tensors."""
    B, S, H, D = q_raw.shape
    Lmax = k_cache_raw.shape[1]
    pos = np.asarray(pos, np.int32)
    kpos = np.broadcast_to(np.arange(Lmax, dtype=np.int32), (B, Lmax))
    if quantized:
        q8, qs, _ = indexer_prepare(q_raw, pos[..., None], cos, sin, bf16_input)
        k8, ks, _ = indexer_prepare(k_cache_raw, kpos, cos, sin, bf16_input)
        qv = dequantize(q8, qs)
        kv = dequantize(k8, ks)
    else:
        q8 = qs = k8 = ks = None
        qv = rope(q_raw, pos[..., None], cos, sin, 64, False, bf16_input).astype(np.float64)
        kv = rope(k_cache_raw, kpos, cos, sin, 64, False, bf16_input).astype(np.float64)
    n_valid = pos + 1
    scores = indexer_scores(qv, w, kv, n_valid)
    idx = topk(np.nan_to_num(scores, nan=0.0), n_valid, K)
    out, lse = sparse_mla(q_mla, latent, kpe, idx, scale)
    return dict(q8=q8, qs=qs, k8=k8, ks=ks, scores=scores, idx=idx, out=out, lse=lse,
                n_valid=n_valid)
