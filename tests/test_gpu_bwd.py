"""GPU parity of the backward kernels (dQ, dK, dV) against the fp64 oracle, called
through the C-ABI library, on the forward kernel's own O and LSE.

Tolerance (derived from the arithmetic): the kernels round P and dS to bf16 (unit
roundoff u = 2^-8) before the products that accumulate the gradients; D = sum_j P_ij dP_ij
and every other step is fp32.  A gradient element is a sum of such rounded terms, so its
error is a few u times the magnitude of the terms; per tensor the bar is
max|diff| <= GRAD_TOL * max(1, max|ref|) with GRAD_TOL = 1e-2 (about 2.5 u).

At the full workload sizes the oracle computes sampled rows (dQ) and keys (dK, dV),
and one identity that holds at any size is checked on every key/value head: the
weights of an admitted row sum to 1, so sum_j dV_j = sum over the group's rows with
keys of dO_i, within u * sum |dO_i| (bf16 rounding of P)."""
import numpy as np
import pytest

import oracle
from block_sparse_flash_csr_amd import api
from block_sparse_flash_csr_amd import workloads as W

from gpu_helpers import dev_bf16, sample_rows, say

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
    dq, dk, dv = api.attn_bwd(q, k, v, g, lse, plan, scale)
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


def test_few_keys_large_scale_bwd():
    """Rows of one to five keys at scale 0.28 (436 queries, 28 keys, d 64): P sits on few
    keys, so any error in D enters dS almost undamped.  Forming D from the forward's bf16 O
    put dK at 1.18e-2 of max|ref| here (the bar is 1e-2); D = sum_j P_ij dP_ij removes that
    term."""
    heads = [(1, 1), (2, 1), (2, 2), (4, 2), (3, 3), (8, 2), (6, 1)]
    rng = np.random.default_rng(888_445)
    sq, sk = int(rng.integers(1, 800)), int(rng.integers(1, 800))
    hq, hkv = heads[int(rng.integers(0, len(heads)))]
    d = (64, 128)[int(rng.integers(0, 2))]
    slices = W.random_slices(rng, sq, sk, int(rng.integers(0, 10)))
    if rng.random() < 0.4:
        slices.append((0, sq, 0, sk, int(rng.integers(0, 2))))
    scale = float(rng.uniform(0.03, 0.3))
    qb, kb, vb = W.random_inputs(rng, sq, sk, hq, hkv, d)
    gb = W.random_grad(rng, sq, hq, d)
    assert (sq, sk, d) == (436, 28, 64) and abs(scale - 0.2809) < 1e-3
    what = f"few keys, scale {scale:.3f}: sq={sq} sk={sk} hq={hq} hkv={hkv} d={d} slices={len(slices)}"
    say(what)
    got = run_bwd(qb, kb, vb, gb, slices, scale)
    check_grads(got, oracle.attn_bwd(qb, kb, vb, gb, slices, scale), what)


def test_causal_s256_bwd():
    w = W.causal_s256()
    full_check(w.q, w.k, w.v, w.slices, w.scale, "bwd causal S=256 d=64")


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


# ---------------------------------------------------------------------------
# full workload sizes, in the forward's launch configuration: sampled outputs
# ---------------------------------------------------------------------------
U_BF16 = 2.0 ** -8


def full_size_run(w, plan, seed):
    import torch
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    gb = W.random_grad(np.random.default_rng(seed), w.sq, w.hq, w.d)
    g = dev_bf16(gb)
    say(f"{w.name}: forward + backward")
    o, lse = api.attn_fwd(q, k, v, plan, w.scale)
    dq, dk, dv = api.attn_bwd(q, k, v, g, lse, plan, w.scale)
    torch.cuda.synchronize()
    for name, t in (("dQ", dq), ("dK", dk), ("dV", dv)):
        assert torch.isfinite(t).all().item(), f"non-finite {name}"
    return gb, lse, dq, dk, dv


def check_dv_sum_identity(w, gb, lse, dv, what):
    """sum_j dV[j, g] == sum over h in g, rows i with keys, of dO[i, h]."""
    import torch
    group = w.hq // w.hkv
    has_keys = torch.isfinite(lse).cpu().numpy()          # [hq, sq]
    do = W.bf16_to_f32(gb).astype(np.float64)             # [sq, hq, d]
    lhs = dv.double().sum(dim=0).cpu().numpy()            # [hkv, d]
    worst = 0.0
    for gi in range(w.hkv):
        rhs = np.zeros(w.d)
        bound = np.zeros(w.d)
        for h in range(gi * group, (gi + 1) * group):
            m = has_keys[h]
            rhs += do[m, h].sum(axis=0)
            bound += np.abs(do[m, h]).sum(axis=0)
        err = np.abs(lhs[gi] - rhs)
        worst = max(worst, float(np.max(err / (U_BF16 * bound + 1e-6))))
        assert np.all(err <= U_BF16 * bound + 1e-6), f"{what}: sum_j dV off for kv head {gi}"
    say(f"{what}: sum_j dV identity holds, worst error {worst:.3f} of the bound")


def test_varlen_causal_t16384_bwd_sampled():
    import torch
    w = W.varlen_causal_t16384()
    plan = api.plan_from_workload(w)
    gb, lse, dq, dk, dv = full_size_run(w, plan, 2002)
    cu = [int(x) for x in w.cu_seqlens]
    extra = cu[:-1] + [c + 1 for c in cu[:-1]] + [c - 1 for c in cu[1:]]
    rows = sample_rows(w, 40, 22, extra)
    rng = np.random.default_rng(23)
    lens = np.diff(cu)
    short = [cu[t] for t in np.argsort(lens)[:2]]                 # first keys of the shortest documents
    kj = sorted(set([c - 1 for c in cu[1:]] + short + [c + 5 for c in short]
                    + [int(x) for x in rng.integers(0, w.sk, 4)]))
    keys = [(int(rng.integers(0, w.hkv)), j) for j in kj]
    say(f"varlen causal t16384 backward: oracle on {len(rows)} rows and {len(keys)} keys")
    rq, rk, rv = oracle.attn_bwd_sampled(w.q, w.k, w.v, gb, w.slices, w.scale, rows=rows, keys=keys)
    r = np.array(rows, np.int64)
    gq = dq[torch.from_numpy(r[:, 1]).cuda(), torch.from_numpy(r[:, 0]).cuda()].cpu().numpy()
    kk = np.array(keys, np.int64)
    ki, kg = torch.from_numpy(kk[:, 1]).cuda(), torch.from_numpy(kk[:, 0]).cuda()
    gk, gv = dk[ki, kg].cpu().numpy(), dv[ki, kg].cpu().numpy()
    check_grads((gq, gk, gv), (rq, rk, rv), "varlen causal t16384 backward sampled")
    check_dv_sum_identity(w, gb, lse, dv, "varlen causal t16384 backward")
    plan.close()


def test_range_slices_s65536_bwd_rows_and_identity():
    """GQA 32/8 at 65536 tokens: sampled dQ rows and the dV identity on every kv head
    (a sampled key there would cost the oracle tens of seconds)."""
    import torch
    w = W.range_slices_s65536()
    plan = api.plan_from_workload(w)
    gb, lse, dq, dk, dv = full_size_run(w, plan, 2004)
    extra = [s[0] for s in w.slices[16:30]] + [s[1] - 1 for s in w.slices[16:30]]
    rows = sample_rows(w, 24, 44, extra)
    rq, _, _ = oracle.attn_bwd_sampled(w.q, w.k, w.v, gb, w.slices, w.scale, rows=rows)
    r = np.array(rows, np.int64)
    gq = dq[torch.from_numpy(r[:, 1]).cuda(), torch.from_numpy(r[:, 0]).cuda()].cpu().numpy()
    err = float(np.max(np.abs(gq - rq)))
    mag = float(np.max(np.abs(rq)))
    say(f"range slices s65536 backward sampled: max|ddQ| = {err:.3e} (max|ref| {mag:.2e})")
    assert err <= GRAD_TOL * max(1.0, mag)
    check_dv_sum_identity(w, gb, lse, dv, "range slices s65536 backward")
    plan.close()


def test_bwd_on_a_plan_with_split_rows():
    """Few queries against long keys: the forward splits every row into parts (merged by
    its second kernel); the backward runs over whole CSR rows and columns regardless."""
    sq, sk, hq, hkv, d = 200, 9000, 4, 2, 128
    rng = np.random.default_rng(43)
    slices = [(0, sq, 0, sk, 1)] + W.random_slices(rng, sq, sk, 3)
    qb, kb, vb = W.random_inputs(rng, sq, sk, hq, hkv, d)
    plan = api.Plan.from_slices(slices, sq, sk, hq, hkv, d)
    assert plan.info()["n_splits"] > 0
    plan.upload()
    gb = W.random_grad(np.random.default_rng(44), sq, hq, d)
    say(f"bwd on a split plan: sq={sq} sk={sk} splits={plan.info()['n_splits']}")
    got = run_bwd(qb, kb, vb, gb, slices, 0.088, plan=plan)
    plan.close()
    check_grads(got, oracle.attn_bwd(qb, kb, vb, gb, slices, 0.088), "bwd split plan")
