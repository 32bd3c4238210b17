"""Seeded synthetic inputs for the sparse-attention hot path.

This module draws random numbers and lays them out; it performs none of the
method's arithmetic (no RoPE, no quantisation, no scores). Both the GPU
path's tests/benchmark and the CPU oracle consume what it returns, so it is
the only code the two sides share.

Every tensor is drawn with numpy's PCG64 generator from the config's seed,
in a fixed order, as float32 N(0, 1) unless stated otherwise. bfloat16
tensors are returned as uint16 bit patterns (round-to-nearest-even from the
float32 draw, done by PyTorch's CPU cast).

Workloads (the shapes the method runs at):
  tiny      B=1, one query at position 255, 256 cached keys, 4 indexer heads,
            top-32, 8 attention heads; indexer in float32 (no FP8 rounding).
  decode16k B=1, position 16383 (16384 keys), 64 indexer heads, top-2048,
            128 attention heads, bf16 q/k activations quantised to FP8.
  batch32   B=32 rows, row b has L_b ~ U{2048..16384} keys (drawn first),
            Lmax = 16384; otherwise as decode16k.
  prefill4k B=1, T=4096 queries at positions 0..4095 against 4096 keys.
  decode128k B=4, position 131071, YaRN rotary table; otherwise as decode16k.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

D_INDEX = 128       # indexer head dim
ROPE_INDEX = 64     # rotated features of an indexer row
D_LATENT = 512      # latent features per cached position
D_ROPE = 64         # rotary-key features per cached position
D_QK_HEAD = 192     # qk_nope (128) + qk_rope (64): the softmax scale's head dim


@dataclass
class Workload:
    name: str
    seed: int
    B: int
    S: int
    H: int            # indexer heads
    Hq: int           # attention heads
    K: int            # top-k budget
    Lmax: int
    lengths: list = field(default_factory=list)   # per batch row: cached keys incl. the new one
    prefill: bool = False
    yarn: bool = False
    fp8: bool = True
    act_bf16: bool = True   # indexer q/k activations are bf16
    w_scale: float = 1.0
    softmax_scale: float = D_QK_HEAD ** -0.5


def mscale_sq(rope_factor: float = 40.0, mscale: float = 1.0) -> float:
    """Square of the YaRN attention-scale correction m = 1 + 0.1*mscale*ln(factor)."""
    m = 0.1 * mscale * math.log(rope_factor) + 1.0
    return m * m


def workload(name: str) -> Workload:
    if name == "tiny":
        return Workload("tiny", 0, B=1, S=1, H=4, Hq=8, K=32, Lmax=256, lengths=[256],
                        fp8=False, act_bf16=False, w_scale=4 ** -0.5)
    if name == "decode16k":
        return Workload("decode16k", 1, B=1, S=1, H=64, Hq=128, K=2048, Lmax=16384,
                        lengths=[16384], w_scale=64 ** -0.5 * 128 ** -0.5)
    if name == "batch32":
        rng = np.random.Generator(np.random.PCG64(2))
        lengths = rng.integers(2048, 16384 + 1, size=32).tolist()
        return Workload("batch32", 2, B=32, S=1, H=64, Hq=128, K=2048, Lmax=16384,
                        lengths=lengths, w_scale=64 ** -0.5 * 128 ** -0.5)
    if name == "prefill4k":
        return Workload("prefill4k", 3, B=1, S=4096, H=64, Hq=128, K=2048, Lmax=4096,
                        lengths=[4096], prefill=True, w_scale=64 ** -0.5 * 128 ** -0.5)
    if name == "decode128k":
        return Workload("decode128k", 4, B=4, S=1, H=64, Hq=128, K=2048, Lmax=131072,
                        lengths=[131072] * 4, yarn=True, w_scale=64 ** -0.5 * 128 ** -0.5,
                        softmax_scale=D_QK_HEAD ** -0.5 * mscale_sq())
    raise KeyError(name)


WORKLOADS = ("tiny", "decode16k", "batch32", "prefill4k", "decode128k")


def sweep_workload(B: int) -> Workload:
    """Supplementary batch sweep: decode16k's shapes with B rows, every row at
    L = 16384 (seed 5)."""
    return Workload(f"sweep-b{B}", 5, B=B, S=1, H=64, Hq=128, K=2048, Lmax=16384,
                    lengths=[16384] * B, w_scale=64 ** -0.5 * 128 ** -0.5)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def positions(wl: Workload) -> np.ndarray:
    """pos [B, S] int32: the position of every query row."""
    if wl.prefill:
        return np.broadcast_to(np.arange(wl.S, dtype=np.int32), (wl.B, wl.S)).copy()
    return np.array([[L - 1] for L in wl.lengths], dtype=np.int32).reshape(wl.B, wl.S)


def make_inputs(wl: Workload, rows_cap: int | None = None) -> dict:
    """Draw every input of one step of the hot path.

    Returns float32 arrays for the indexer activations (q_raw [B,S,H,128],
    k_raw [B,Lmax,128]: key at position p of batch b is k_raw[b, p]) -- these
    hold bf16-representable values when the workload's activations are bf16 --
    w [B,S,H], and bf16 bit patterns for the attention inputs q_mla
    [B,S,Hq,576], latent [B,Lmax,512], kpe [B,Lmax,64]."""
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    if wl.name == "batch32":
        rng.integers(2048, 16384 + 1, size=32)      # the lengths are the first draw
    B, S, H, Hq, L = wl.B, wl.S, wl.H, wl.Hq, wl.Lmax
    q_raw = rng.standard_normal((B, S, H, D_INDEX), dtype=np.float32)
    k_raw = rng.standard_normal((B, L, D_INDEX), dtype=np.float32)
    w = rng.standard_normal((B, S, H), dtype=np.float32) * np.float32(wl.w_scale)
    q_mla = rng.standard_normal((B, S, Hq, D_LATENT + D_ROPE), dtype=np.float32)
    latent = rng.standard_normal((B, L, D_LATENT), dtype=np.float32)
    kpe = rng.standard_normal((B, L, D_ROPE), dtype=np.float32)
    if wl.act_bf16:
        q_raw = bf16_bits_to_f32(to_bf16_bits(q_raw))
        k_raw = bf16_bits_to_f32(to_bf16_bits(k_raw))
    return dict(
        pos=positions(wl), q_raw=q_raw, k_raw=k_raw, w=w.astype(np.float32),
        q_mla=to_bf16_bits(q_mla), latent=to_bf16_bits(latent), kpe=to_bf16_bits(kpe),
    )


# ----------------------------------------------------------- unit inputs --

def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def topk_scores(seed: int, rows: int, L: int, kind: str = "normal") -> np.ndarray:
    """float32 [rows, L] score rows for exercising a top-k.

    kind: normal (continuous), ties (values from a small integer set, many
    exact ties), zeros (+0/-0 mixed), constant (all equal), wide (mixed
    magnitudes and signs, including huge and tiny values)."""
    g = rng(seed)
    if kind == "normal":
        return g.standard_normal((rows, L), dtype=np.float32)
    if kind == "ties":
        return g.integers(-8, 8, size=(rows, L)).astype(np.float32) * np.float32(0.25)
    if kind == "zeros":
        s = np.where(g.random((rows, L)) < 0.5, np.float32(0.0), np.float32(-0.0))
        bump = g.random((rows, L)) < 0.05
        return np.where(bump, g.standard_normal((rows, L), dtype=np.float32), s).astype(np.float32)
    if kind == "constant":
        return np.full((rows, L), 1.5, np.float32)
    if kind == "wide":
        mag = np.exp2(g.integers(-120, 120, size=(rows, L)).astype(np.float32))
        sign = np.where(g.random((rows, L)) < 0.5, -1.0, 1.0).astype(np.float32)
        return (mag * sign * g.random((rows, L), dtype=np.float32)).astype(np.float32)
    raise KeyError(kind)


def random_selection(seed: int, rows: int, K: int, n_valid, fill: float = 1.0) -> np.ndarray:
    """int32 [rows, K]: per row, a random set of distinct positions below
    n_valid[r] of size min(K, round(fill*n_valid)), in random order, padded
    with -1 at random slots."""
    g = rng(seed)
    nv = np.broadcast_to(np.asarray(n_valid), (rows,))
    out = np.full((rows, K), -1, np.int32)
    for r in range(rows):
        n = int(nv[r])
        take = min(K, max(0, int(round(fill * n))))
        sel = g.choice(n, size=take, replace=False).astype(np.int32) if take else np.empty(0, np.int32)
        slots = g.choice(K, size=take, replace=False)
        out[r, slots] = sel
    return out
