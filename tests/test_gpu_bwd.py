"""GPU parity of the backward kernels (dQ, dK, dV) against the fp64 oracle, called
through the C-ABI library, on the forward kernel's own O and LSE.

Tolerance (derived from the arithmetic): the kernels round P and dS to bf16 (unit
roundoff 2^-9) before the products that accumulate the gradients, and D = rowsum(dO*O)
takes O as the forward's bf16 output; every other step is fp32.  Per tensor the bar is
max|diff| <= GRAD_TOL * max(1, max|reference|)."""
import numpy as np
import pytest

import oracle
from block_sparse_flash_csr_amd import api
from block_sparse_flash_csr_amd import workloads as W

from gpu_helpers import dev_bf16, say

pytestmark = pytest.mark.gpu

GRAD_TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    api.library()
    yield
    torch.cuda.synchronize()


def run_bwd(qb, kb, vb, gb, slices, scale, plan=None):
    import torch
    sq, hq, d = qb.shape
    sk, hkv, _ = kb.shape
    q, k, v, g = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(gb)
    own = plan is None
    if own:
        plan = api.Plan.from_slices(slices, sq, sk, hq, hkv, d).upload()
    o, lse = api.attn_fwd(q, k, v, plan, scale)
    dq, dk, dv = api.attn_bwd(q, k, v, o, g, lse, plan, scale)
    torch.cuda.synchronize()
    out = dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()
    if own:
        plan.close()
    return out


def check_grads(got, ref, what):
    errs = []
    for name, x, r in zip(("dQ", "dK", "dV"), got, ref):
        x = x.astype(np.float64)
        assert np.isfinite(x).all(), f"{what}: non-finite {name}"
        err = float(np.max(np.abs(x - r))) if r.size else 0.0
        mag = float(np.max(np.abs(r))) if r.size else 0.0
        errs.append((name, err, mag))
    say(f"{what}: " + ", ".join(f"max|d{n}| = {e:.3e} (max|ref| {m:.2e})" for n, e, m in errs))
    for name, err, mag in errs:
        assert err <= GRAD_TOL * max(1.0, mag), f"{what}: {name} error {err} (max|ref| {mag})"


def full_check(qb, kb, vb, slices, scale, what, seed=0):
    sq, hq, d = qb.shape
    sk, hkv, _ = kb.shape
    gb = W.random_grad(np.random.default_rng(1000 + seed), sq, hq, d)
    say(f"{what}: sq={sq} sk={sk} hq={hq} hkv={hkv} d={d} slices={len(slices)}")
    got = run_bwd(qb, kb, vb, gb, slices, scale)
    ref = oracle.attn_bwd(qb, kb, vb, gb, slices, scale)
    check_grads(got, ref, what)
    return got, ref


def test_config1_bwd():
    w = W.config1()
    full_check(w.q, w.k, w.v, w.slices, w.scale, "bwd config1 causal S=256 d=64")


@pytest.mark.parametrize("seed,sq,sk,hq,hkv,d,n", [
    (1, 300, 300, 2, 2, 128, 4),
    (2, 517, 389, 4, 2, 128, 6),
    (3, 640, 640, 2, 1, 64, 3),
    (4, 129, 700, 2, 2, 128, 8),
    (5, 700, 129, 3, 3, 64, 5),
    (6, 1, 50, 1, 1, 128, 2),
    (7, 260, 260, 8, 1, 128, 4),
])
def test_bwd_random_masks(seed, sq, sk, hq, hkv, d, n):
    rng = np.random.default_rng(seed)
    slices = W.random_slices(rng, sq, sk, n)
    qb, kb, vb = W.random_inputs(rng, sq, sk, hq, hkv, d)
    full_check(qb, kb, vb, slices, 1.0 / np.sqrt(d), f"bwd random seed={seed}", seed)


def test_bwd_partial_offsets_and_ragged_rows():
    sq, sk, d = 400, 400, 128
    rng = np.random.default_rng(77)
    qb, kb, vb = W.random_inputs(rng, sq, sk, 2, 1, d)
    slices = [(0, sq, 0, sk - 61, 1), (3, 131, 200, 333, 1), (150, 151, 0, 400, 0)]
    full_check(qb, kb, vb, slices, 1.0 / np.sqrt(d), "bwd partial offsets", 1)
    slices = [(q0, q0 + 1, 0, min(sk, q0 + 1 + (q0 % 7)), 0) for q0 in range(0, sq)]
    full_check(qb, kb, vb, slices, 1.0 / np.sqrt(d), "bwd per-row ragged windows", 2)


def test_bwd_masked_rows_and_empty_mask():
    sq, sk, d = 384, 256, 128
    rng = np.random.default_rng(10)
    qb, kb, vb = W.random_inputs(rng, sq, sk, 2, 2, d)
    slices = [(0, 128, 0, 256, 1), (256, 384, 100, 140, 1)]
    got, _ = full_check(qb, kb, vb, slices, 0.1, "bwd masked rows", 3)
    assert np.all(got[0][128:256] == 0), "rows without keys have dQ = 0"
    # no query reaches keys 140..255 (the causal slice keeps its bottom-right diagonal:
    # row i of (256, 384, 100, 140) sees keys up to i - 244)
    slices = [(0, 128, 0, 100, 0), (256, 384, 100, 140, 1)]
    got, _ = full_check(qb, kb, vb, slices, 0.1, "bwd unreached keys", 6)
    assert np.all(got[1][140:] == 0) and np.all(got[2][140:] == 0), "unreached keys have dK = dV = 0"
    got, _ = full_check(qb, kb, vb, [], 0.1, "bwd empty mask", 4)
    assert all(np.all(g == 0) for g in got)


def test_bwd_varlen_causal_documents():
    rng = np.random.default_rng(21)
    lens = [37, 300, 129, 1, 200, 180]
    cu, slices = W.varlen_slices(lens)
    s = int(cu[-1])
    qb, kb, vb = W.random_inputs(rng, s, s, 4, 2, 128)
    full_check(qb, kb, vb, slices, 1.0 / np.sqrt(128), "bwd varlen causal", 5)


def test_bwd_deterministic():
    import torch
    rng = np.random.default_rng(31)
    sq = sk = 500
    slices = W.random_slices(rng, sq, sk, 5)
    qb, kb, vb = W.random_inputs(rng, sq, sk, 4, 2, 128)
    gb = W.random_grad(rng, sq, 4, 128)
    a = run_bwd(qb, kb, vb, gb, slices, 0.09)
    b = run_bwd(qb, kb, vb, gb, slices, 0.09)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
