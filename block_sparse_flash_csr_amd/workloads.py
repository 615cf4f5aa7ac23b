"""Seeded synthetic workloads: mask descriptions and bf16 Q/K/V.

This module holds no attention arithmetic.  It draws mask parameters and
inputs from ``numpy.random.default_rng(seed)`` (PCG64) and is the one module that
both the GPU tests and the oracle tests take their inputs from.

Draw order for every workload: mask parameters first, then
``standard_normal(float32)`` for Q, then K, then V, each rounded to bf16
(round to nearest even).

Mask vocabulary (slices): ``(q0, q1, k0, k1, type)`` with type 0 = full
rectangle, 1 = causal inside the rectangle, aligned at its bottom-right corner
(pair (i, j) admitted iff ``j - k1 <= i - q1``).  The workloads follow the
pages' mask families: varlen causal (MagiAttention v1.1.0 news, kernel benchmark
paragraph), the strided block-sparse pattern (UltraAttn blog, 1 and 8) and
flexible range slices with full/causal types (MagiAttention news, flexible mask
list).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

FULL, CAUSAL = 0, 1


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.  Finite inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    """One attention problem: shapes, a slice mask (or a varlen / block form) and inputs."""
    name: str
    sq: int
    sk: int
    hq: int
    hkv: int
    d: int
    slices: list                      # list of (q0, q1, k0, k1, type)
    scale: float
    seed: int
    cu_seqlens: np.ndarray | None = None   # varlen form (int32 [n_docs + 1])
    block_codes: np.ndarray | None = None  # block form (uint8 [nbq, nbk]; 0 empty 1 full 2 causal)
    block: tuple | None = None             # (block_q, block_k) of block_codes
    q: np.ndarray | None = field(default=None, repr=False)  # uint16 [sq, hq, d]
    k: np.ndarray | None = field(default=None, repr=False)  # uint16 [sk, hkv, d]
    v: np.ndarray | None = field(default=None, repr=False)
    extra: dict = field(default_factory=dict)


def _draw_qkv(rng, sq, sk, hq, hkv, d):
    q = bf16_bits(rng.standard_normal((sq, hq, d), dtype=np.float32))
    k = bf16_bits(rng.standard_normal((sk, hkv, d), dtype=np.float32))
    v = bf16_bits(rng.standard_normal((sk, hkv, d), dtype=np.float32))
    return q, k, v


def varlen_lengths(rng, total: int, n_docs: int, lo: int, hi: int) -> list:
    """Document lengths drawn U[lo, hi), rescaled to sum to ``total``.

    L_i = floor(u_i * total / sum(u)); the rounding remainder goes to the last
    document, so a rescaled length may fall slightly outside [lo, hi].
    """
    u = rng.uniform(lo, hi, size=n_docs)
    lens = [int(np.floor(x * total / u.sum())) for x in u]
    lens[-1] += total - sum(lens)
    return lens


def varlen_slices(lens) -> tuple:
    cu = np.zeros(len(lens) + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    slices = [(int(cu[i]), int(cu[i + 1]), int(cu[i]), int(cu[i + 1]), CAUSAL)
              for i in range(len(lens)) if cu[i + 1] > cu[i]]
    return cu, slices


def strided_block_codes(n_blocks: int, stride: int) -> np.ndarray:
    """First KV block column + causal block diagonal + every stride-th diagonal below it."""
    codes = np.zeros((n_blocks, n_blocks), np.uint8)
    for i in range(n_blocks):
        for j in range(i + 1):
            if i == j:
                codes[i, j] = 2
            elif j == 0 or (i - j) % stride == 0:
                codes[i, j] = 1
    return codes


def block_slices(codes: np.ndarray, bq: int, bk: int, sq: int, sk: int) -> list:
    out = []
    for i, j in zip(*np.nonzero(codes)):
        q0, k0 = int(i) * bq, int(j) * bk
        q1, k1 = min(q0 + bq, sq), min(k0 + bk, sk)
        out.append((q0, q1, k0, k1, FULL if codes[i, j] == 1 else CAUSAL))
    return out


def range_slice_mask(rng, s: int, n_frames: int, frame: int, n_seeded: int, qblk: int) -> list:
    """Video-frame full slices plus seeded (q_range, k_range, full|causal) slices.

    Frames: (f*frame, (f+1)*frame) x same, full.  Seeded slice i covers queries
    [qa, qb) = [qblk*i, qblk*(i+1)); width W = max(1, floor(u*qb)), u ~ U(0.2, 0.4);
    a coin t in {0, 1}; causal (qa, qb, qb-W, qb) when i == 0 or t == 0 or qa < W,
    else full (qa, qb, k0, k0+W) with k0 = floor(v*(qa-W)), v ~ U(0, 1).
    """
    slices = [(f * frame, (f + 1) * frame, f * frame, (f + 1) * frame, FULL)
              for f in range(n_frames)]
    for i in range(n_seeded):
        qa, qb = qblk * i, qblk * (i + 1)
        u = rng.uniform(0.2, 0.4)
        w = max(1, int(np.floor(u * qb)))
        t = int(rng.integers(0, 2))
        if i == 0 or t == 0 or qa < w:
            slices.append((qa, qb, qb - w, qb, CAUSAL))
        else:
            v = rng.uniform(0.0, 1.0)
            k0 = int(np.floor(v * (qa - w)))
            slices.append((qa, qb, k0, k0 + w, FULL))
    assert qblk * n_seeded <= s
    return slices


# ----------------------------------------------------------------------------
# The five workloads
# ----------------------------------------------------------------------------

def causal_s256(with_inputs: bool = True) -> Workload:
    """Single-sequence causal: batch 1, 2 heads, S = 256, d = 64, scale 1/8 (seed 1)."""
    rng = np.random.default_rng(1)
    s, h, d = 256, 2, 64
    w = Workload("causal_s256_h2_d64", s, s, h, h, d, [(0, s, 0, s, CAUSAL)], 1.0 / np.sqrt(d), 1)
    if with_inputs:
        w.q, w.k, w.v = _draw_qkv(rng, s, s, h, h, d)
    return w


def varlen_causal_t16384(with_inputs: bool = True) -> Workload:
    """Varlen causal: 16384 packed tokens, 8 documents U[512, 4096) rescaled, 16 heads, d 128."""
    rng = np.random.default_rng(2)
    total, h, d = 16384, 16, 128
    lens = varlen_lengths(rng, total, 8, 512, 4096)
    cu, slices = varlen_slices(lens)
    w = Workload("varlen_causal_t16384_docs8_h16_d128", total, total, h, h, d, slices,
                 1.0 / np.sqrt(d), 2, cu_seqlens=cu, extra={"lengths": lens})
    if with_inputs:
        w.q, w.k, w.v = _draw_qkv(rng, total, total, h, h, d)
    return w


def block_sparse_strided_s32768(with_inputs: bool = True) -> Workload:
    """Block-sparse strided: S = 32768, 128x128 blocks, column 0 + causal diagonal + every
    8th diagonal below it; 16 heads, d 128 (seed 3)."""
    rng = np.random.default_rng(3)
    s, h, d, b = 32768, 16, 128, 128
    codes = strided_block_codes(s // b, 8)
    w = Workload("block_sparse_strided_s32768_b128_h16_d128", s, s, h, h, d,
                 block_slices(codes, b, b, s, s), 1.0 / np.sqrt(d), 3, block_codes=codes,
                 block=(b, b))
    if with_inputs:
        w.q, w.k, w.v = _draw_qkv(rng, s, s, h, h, d)
    return w


def range_slices_s65536(with_inputs: bool = True) -> Workload:
    """Range slices: S = 65536, 16 full 4096-token frames + 64 seeded slices; GQA 32/8, d 128."""
    rng = np.random.default_rng(4)
    s, hq, hkv, d = 65536, 32, 8, 128
    slices = range_slice_mask(rng, s, 16, 4096, 64, 1024)
    w = Workload("range_slices_s65536_gqa32x8_d128", s, s, hq, hkv, d, slices, 1.0 / np.sqrt(d), 4)
    if with_inputs:
        w.q, w.k, w.v = _draw_qkv(rng, s, s, hq, hkv, d)
    return w


def kv_split_q8192(with_inputs: bool = True, q_chunk: int = 7) -> Workload:
    """KV-split share: a Q chunk of 8192 tokens at global chunk ``q_chunk`` against 8 KV
    chunks of 8192 tokens, causal over the 65536 global positions; 32 heads, d 128 (seed 5).

    ``slices`` is the unsplit mask in chunk-local query coordinates against global
    keys: queries [0, 8192) are global positions [8192*q_chunk, ...).  ``extra['chunk_slices']``
    holds the per-KV-chunk masks (chunk-local on both axes).
    """
    rng = np.random.default_rng(5)
    c, n_chunks, h, d = 8192, 8, 32, 128
    q_lo = c * q_chunk
    # unsplit: query i (global q_lo + i) sees keys j <= q_lo + i
    slices = [(0, c, 0, q_lo + c, CAUSAL)]
    chunk_slices = []
    for kc in range(n_chunks):
        if kc < q_chunk:
            chunk_slices.append([(0, c, 0, c, FULL)])
        elif kc == q_chunk:
            chunk_slices.append([(0, c, 0, c, CAUSAL)])
        else:
            chunk_slices.append([])
    w = Workload("kv_split_q8192_x8chunks_h32_d128", c, c * n_chunks, h, h, d, slices,
                 1.0 / np.sqrt(d), 5, extra={"chunk": c, "n_chunks": n_chunks, "q_chunk": q_chunk,
                                             "chunk_slices": chunk_slices})
    if with_inputs:
        w.q, w.k, w.v = _draw_qkv(rng, c, c * n_chunks, h, h, d)
    return w


WORKLOADS = {1: causal_s256, 2: varlen_causal_t16384, 3: block_sparse_strided_s32768, 4: range_slices_s65536, 5: kv_split_q8192}


def random_slices(rng, sq: int, sk: int, n: int, allow_empty: bool = True) -> list:
    """Small random slice lists for tests: unaligned, overlapping, both types."""
    out = []
    for _ in range(n):
        q0 = int(rng.integers(0, sq))
        q1 = int(rng.integers(q0 if allow_empty else q0 + 1, sq + 1))
        k0 = int(rng.integers(0, sk))
        k1 = int(rng.integers(k0 if allow_empty else k0 + 1, sk + 1))
        out.append((q0, q1, k0, k1, int(rng.integers(0, 2))))
    return out


def random_inputs(rng, sq: int, sk: int, hq: int, hkv: int, d: int):
    return _draw_qkv(rng, sq, sk, hq, hkv, d)


def device_normal_bf16(shape, seed: int):
    """Standard normal bf16 tensor drawn on the current GPU by torch's seeded generator
    (for inputs too large to draw on the host; tests copy back the parts they check)."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.bfloat16)


def doc_lengths(rng, total: int, lo: int, hi: int):
    """Document lengths drawn uniformly in [lo, hi) until they cover `total` tokens; the
    last one is cut to fit (at least 1 token)."""
    out, n = [], 0
    while n < total:
        L = min(int(rng.integers(lo, hi)), total - n)
        out.append(L)
        n += L
    return out


def random_grad(rng, sq: int, hq: int, d: int):
    """Upstream gradient dO [sq, hq, d]: standard normal, as bf16 bit patterns."""
    return bf16_bits(rng.standard_normal((sq, hq, d), dtype=np.float32))
