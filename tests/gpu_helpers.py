"""Shared helpers of the GPU parity tests: device tensors from the seeded bf16 bits,
row sampling, and the comparison against the fp64 oracle at the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np

from block_sparse_flash_csr_amd import workloads as W

O_TOL = 1e-2      # max |dO| against the fp64 oracle
LSE_TOL = 1e-3    # max |dLSE| against the fp64 oracle


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def host_bits(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_floor(o_ref: np.ndarray) -> float:
    """Largest error that rounding the exact output to bf16 alone would cause."""
    r = W.bf16_to_f32(W.bf16_bits(o_ref.astype(np.float32))).astype(np.float64)
    return float(np.max(np.abs(r - o_ref))) if o_ref.size else 0.0


def compare(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray,
            what: str):
    """o_*: [..., d]; lse_*: matching leading shape.  Asserts the tolerances."""
    o_gpu = o_gpu.astype(np.float64)
    lse_gpu = lse_gpu.astype(np.float64)
    inf_ref = np.isneginf(lse_ref)
    assert not np.isnan(o_gpu).any(), f"{what}: NaN in O"
    assert not np.isnan(lse_gpu).any(), f"{what}: NaN in LSE"
    assert np.array_equal(np.isneginf(lse_gpu), inf_ref), f"{what}: -inf rows differ"
    assert np.all(o_gpu[inf_ref] == 0), f"{what}: rows without keys must be 0"
    do = float(np.max(np.abs(o_gpu - o_ref))) if o_ref.size else 0.0
    fin = ~inf_ref
    dl = float(np.max(np.abs(lse_gpu[fin] - lse_ref[fin]))) if fin.any() else 0.0
    say(f"{what}: max|dO| = {do:.3e} (bf16 output floor {bf16_floor(o_ref):.3e}), "
        f"max|dLSE| = {dl:.3e}")
    assert do <= O_TOL, f"{what}: max|dO| {do} > {O_TOL}"
    assert dl <= LSE_TOL, f"{what}: max|dLSE| {dl} > {LSE_TOL}"
    return do, dl


def sample_rows(w, n_random: int, seed: int, extra_rows=()):
    """(h, i) pairs: seeded random rows plus structural rows (ends, tile edges, extras)."""
    rng = np.random.default_rng(seed)
    rows = set()
    hs = rng.integers(0, w.hq, size=n_random)
    is_ = rng.integers(0, w.sq, size=n_random)
    rows.update(zip(hs.tolist(), is_.tolist()))
    edge = {0, 1, w.sq - 1, min(127, w.sq - 1), min(128, w.sq - 1)}
    edge.update(int(x) for x in extra_rows if 0 <= x < w.sq)
    for i in edge:
        rows.add((0, i))
        rows.add((w.hq - 1, i))
    return sorted(rows)
