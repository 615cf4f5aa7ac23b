"""The backward given the forward's fp32 output (bsfa_attn_bwd_o32): D_i = dO_i . O_i is
formed from that O inside the dQ kernel instead of by the separate D pass.

Against the fp64 oracle at the gradient bar of test_gpu_bwd.py (max|diff| <= 1e-2 *
max(1, max|ref|) per tensor), on the few-key case that breaks the bar when D comes from
the bf16 output, on the backward sweep's cases, on ragged GQA and split-row plans, and
at full size on sampled rows and keys with the sum_j dV identity."""
import numpy as np
import pytest

import oracle
from block_sparse_flash_csr_amd import api
from block_sparse_flash_csr_amd import workloads as W

from gpu_helpers import dev_bf16, sample_rows, say
from test_gpu_bwd import check_dv_sum_identity, check_grads
from test_gpu_sweep import draw_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    api.library()
    yield
    torch.cuda.synchronize()


def run_o32(qb, kb, vb, gb, slices, scale, bk=128):
    """Forward with fp32 O, then the backward from it; (dQ, dK, dV) on the host."""
    import torch
    sq, hq, d = qb.shape
    sk, hkv, _ = kb.shape
    q, k, v, g = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(gb)
    plan = api.Plan.from_slices(slices, sq, sk, hq, hkv, d, bk=bk).upload()
    o, lse = api.attn_fwd(q, k, v, plan, scale, out_dtype=torch.float32)
    dq, dk, dv = api.attn_bwd(q, k, v, g, lse, plan, scale, o=o)
    torch.cuda.synchronize()
    plan.close()
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


def test_bwd_from_fp32_o_few_keys_large_scale():
    """The case where D from the bf16 output put dK at 1.18e-2 of max|ref| (436 queries,
    28 keys, rows of one to five keys, scale 0.28, d 64)."""
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
    assert (sq, sk, d) == (436, 28, 64)
    what = f"bwd from fp32 O, few keys scale {scale:.3f}: sq={sq} sk={sk} hq={hq} hkv={hkv}"
    say(what)
    check_grads(run_o32(qb, kb, vb, gb, slices, scale), oracle.attn_bwd(qb, kb, vb, gb, slices, scale), what)


@pytest.mark.parametrize("seed", range(64))
def test_bwd_from_fp32_o_sweep(seed):
    rng, sq, sk, hq, hkv, d, bk, slices, scale, qb, kb, vb = draw_case(seed)
    gb = W.random_grad(rng, sq, hq, d)
    what = f"bwd from fp32 O sweep seed={seed} sq={sq} sk={sk} hq={hq} hkv={hkv} d={d} slices={len(slices)}"
    say(what)
    check_grads(run_o32(qb, kb, vb, gb, slices, scale), oracle.attn_bwd(qb, kb, vb, gb, slices, scale), what)


@pytest.mark.parametrize("kind", ["gqa_ragged_d64", "split_rows_d128"])
def test_bwd_from_fp32_o_plans(kind):
    rng = np.random.default_rng(77)
    if kind == "gqa_ragged_d64":
        sq, sk, hq, hkv, d = 389, 517, 6, 2, 64
        slices = W.random_slices(rng, sq, sk, 8)
    else:
        sq, sk, hq, hkv, d = 256, 6000, 2, 1, 128
        slices = [(0, sq, 0, sk, 1), (0, 40, 2000, 2100, 0)]
    qb, kb, vb = W.random_inputs(rng, sq, sk, hq, hkv, d)
    gb = W.random_grad(rng, sq, hq, d)
    what = f"bwd from fp32 O {kind}: sq={sq} sk={sk} hq={hq} hkv={hkv} d={d}"
    say(what)
    check_grads(run_o32(qb, kb, vb, gb, slices, 0.1), oracle.attn_bwd(qb, kb, vb, gb, slices, 0.1), what)


def test_bwd_from_fp32_o_masked_rows_and_empty_mask():
    """Rows without keys (O = 0, LSE = -inf, D = 0), keys no query reaches, an empty mask."""
    sq, sk, d = 384, 256, 128
    rng = np.random.default_rng(10)
    qb, kb, vb = W.random_inputs(rng, sq, sk, 2, 2, d)
    cases = [("masked rows", [(0, 128, 0, 256, 1), (256, 384, 100, 140, 1)]),
             ("unreached keys", [(0, 128, 0, 100, 0), (256, 384, 100, 140, 1)]),
             ("empty mask", [])]
    for i, (what, slices) in enumerate(cases):
        gb = W.random_grad(np.random.default_rng(1003 + i), sq, 2, d)
        say(f"bwd from fp32 O, {what}")
        got = run_o32(qb, kb, vb, gb, slices, 0.1)
        check_grads(got, oracle.attn_bwd(qb, kb, vb, gb, slices, 0.1), f"bwd from fp32 O, {what}")
        if what == "masked rows":
            assert np.all(got[0][128:256] == 0), "rows without keys have dQ = 0"
        if what == "unreached keys":
            assert np.all(got[1][140:] == 0) and np.all(got[2][140:] == 0)
        if what == "empty mask":
            assert all(np.all(g == 0) for g in got)


def test_bwd_from_fp32_o_at_full_size():
    """Varlen causal, 16384 tokens, 16 heads, d 128, backward from the fp32 O: sampled dQ
    rows and dK, dV keys against the oracle, the sum_j dV identity, determinism, and D
    against the D pass's.  The two D differ by the forward's bf16 weights: O is the
    weighted average with weights rounded to bf16 (relative 2^-9 each), the D pass sums
    fp32 P dP, so they agree to about 2^-8 of max|D|, not to summation order."""
    import torch
    w = W.varlen_causal_t16384()
    plan = api.plan_from_workload(w)
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    gb = W.random_grad(np.random.default_rng(2002), w.sq, w.hq, w.d)
    g = dev_bf16(gb)
    say(f"{w.name}: backward from fp32 O")
    o32, lse = api.attn_fwd(q, k, v, plan, w.scale, out_dtype=torch.float32)
    d_pass = torch.empty_like(lse)
    d_o32 = torch.empty_like(lse)
    api.attn_bwd(q, k, v, g, lse, plan, w.scale, delta=d_pass)
    dq, dk, dv = api.attn_bwd(q, k, v, g, lse, plan, w.scale, delta=d_o32, o=o32)
    again = api.attn_bwd(q, k, v, g, lse, plan, w.scale, o=o32)
    torch.cuda.synchronize()
    dd = float((d_o32 - d_pass).abs().max())
    dmag = float(d_pass.abs().max())
    say(f"{w.name}: max|D(O) - D(pass)| = {dd:.3e} (max|D| {dmag:.2e})")
    assert dd <= 2.0 ** -8 * max(1.0, dmag), (dd, dmag)
    for name, x, y in zip(("dQ", "dK", "dV"), (dq, dk, dv), again):
        assert torch.isfinite(x).all().item(), name
        assert torch.equal(x, y), f"{name}: not deterministic"
    cu = [int(x) for x in w.cu_seqlens]
    extra = cu[:-1] + [c + 1 for c in cu[:-1]] + [c - 1 for c in cu[1:]]
    rows = sample_rows(w, 40, 22, extra)
    rng = np.random.default_rng(23)
    lens = np.diff(cu)
    short = [cu[t] for t in np.argsort(lens)[:2]]
    kj = sorted(set([c - 1 for c in cu[1:]] + short + [c + 5 for c in short]
                    + [int(x) for x in rng.integers(0, w.sk, 4)]))
    keys = [(int(rng.integers(0, w.hkv)), j) for j in kj]
    say(f"{w.name} backward from fp32 O: oracle on {len(rows)} rows and {len(keys)} keys")
    rq, rk, rv = oracle.attn_bwd_sampled(w.q, w.k, w.v, gb, w.slices, w.scale, rows=rows, keys=keys)
    r = np.array(rows, np.int64)
    gq = dq[torch.from_numpy(r[:, 1]).cuda(), torch.from_numpy(r[:, 0]).cuda()].cpu().numpy()
    kk = np.array(keys, np.int64)
    ki, kg = torch.from_numpy(kk[:, 1]).cuda(), torch.from_numpy(kk[:, 0]).cuda()
    check_grads((gq, dk[ki, kg].cpu().numpy(), dv[ki, kg].cpu().numpy()), (rq, rk, rv),
                f"{w.name} backward from fp32 O sampled")
    check_dv_sum_identity(w, gb, lse, dv, f"{w.name} backward from fp32 O")
    plan.close()
