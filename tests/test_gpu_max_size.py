"""GPU parity at the largest sizes of the suite: 2,097,152 tokens, 8 query heads on one
key/value head, head dim 128, so Q, O and dO are 4 GiB each (bf16) and dQ 8 GiB (fp32):
every kernel address past 2^31 bytes is exercised.  Mask: varlen causal over seeded
documents of 512..1535 tokens.  The inputs are drawn on the GPU by a seeded generator;
the oracle runs on one document at a time (its rows only see its own keys, so the
document alone is the same problem, shifted) for a few documents, the first, the last
and those whose rows lie past the 2^31-byte offset."""
import numpy as np
import pytest

import oracle
from block_sparse_flash_csr_amd import api
from block_sparse_flash_csr_amd import workloads as W

from gpu_helpers import compare, host_bits, say

pytestmark = pytest.mark.gpu

S, HQ, HKV, D = 1 << 21, 8, 1, 128
SCALE = 1.0 / np.sqrt(D)
GRAD_TOL = 1e-2   # max|d| <= GRAD_TOL * max(1, max|ref|), as for the other gradient tests
U_BF16 = 2.0 ** -8


@pytest.fixture(scope="module")
def setup():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    lens = W.doc_lengths(np.random.default_rng(91), S, 512, 1536)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    say(f"max size: S={S} hq={HQ} hkv={HKV} d={D}, {len(lens)} documents; drawing inputs on the GPU")
    q = W.device_normal_bf16((S, HQ, D), 92)
    k = W.device_normal_bf16((S, HKV, D), 93)
    v = W.device_normal_bf16((S, HKV, D), 94)
    plan = api.Plan.from_varlen(cu, HQ, HKV, D, causal=True).upload()
    half = (1 << 31) // (HQ * D * 2)           # first token whose Q row starts at 2^31 bytes
    d_half = int(np.searchsorted(cu, half, side="right")) - 1
    docs = sorted({0, 1, d_half, d_half + 1, len(lens) // 2, len(lens) - 2, len(lens) - 1})
    yield q, k, v, plan, cu, docs
    plan.close()
    del q, k, v
    torch.cuda.empty_cache()


def doc_bits(t, c0, c1):
    return host_bits(t[c0:c1])


def test_max_size_forward(setup):
    import torch
    q, k, v, plan, cu, docs = setup
    say("max size forward: launching")
    o, lse = api.attn_fwd(q, k, v, plan, SCALE)
    torch.cuda.synchronize()
    assert not torch.isnan(o.float()).any().item()
    for di in docs:
        c0, c1 = int(cu[di]), int(cu[di + 1])
        L = c1 - c0
        o_ref, lse_ref = oracle.attn_fwd(doc_bits(q, c0, c1), doc_bits(k, c0, c1), doc_bits(v, c0, c1),
                                         [(0, L, 0, L, 1)], SCALE)
        o_gpu = W.bf16_to_f32(host_bits(o[c0:c1]))
        compare(o_gpu, lse[:, c0:c1].cpu().numpy().T, o_ref, lse_ref.T,
                f"max size forward, document {di} (tokens {c0}..{c1 - 1})")
    del o, lse


def test_max_size_backward(setup):
    import torch
    q, k, v, plan, cu, docs = setup
    g = W.device_normal_bf16((S, HQ, D), 95)
    o, lse = api.attn_fwd(q, k, v, plan, SCALE)
    say("max size backward: launching")
    dq, dk, dv = api.attn_bwd(q, k, v, g, lse, plan, SCALE)
    torch.cuda.synchronize()
    for name, t in (("dQ", dq), ("dK", dk), ("dV", dv)):
        assert torch.isfinite(t).all().item(), f"non-finite {name}"
    for di in docs:
        c0, c1 = int(cu[di]), int(cu[di + 1])
        L = c1 - c0
        rq, rk, rv = oracle.attn_bwd(doc_bits(q, c0, c1), doc_bits(k, c0, c1), doc_bits(v, c0, c1),
                                     doc_bits(g, c0, c1), [(0, L, 0, L, 1)], SCALE)
        msg = []
        for name, gpu, ref in (("dQ", dq[c0:c1], rq), ("dK", dk[c0:c1], rk), ("dV", dv[c0:c1], rv)):
            err = float(np.max(np.abs(gpu.double().cpu().numpy() - ref)))
            mag = float(np.max(np.abs(ref)))
            msg.append(f"{name} {err:.2e} (max|ref| {mag:.2e})")
            assert err <= GRAD_TOL * max(1.0, mag), f"document {di}: {name} {err} (max|ref| {mag})"
        say(f"max size backward, document {di} (tokens {c0}..{c1 - 1}): max|d| " + ", ".join(msg))
    # every key: sum_j dV[j] equals the sum of dO over the rows that see a key (all of them here)
    lhs = torch.sum(dv, dim=0, dtype=torch.float64)[0]
    rhs = torch.sum(g, dim=(0, 1), dtype=torch.float64)
    bound = torch.sum(g.abs(), dim=(0, 1), dtype=torch.float64)
    err = (lhs - rhs).abs()
    assert torch.all(err <= U_BF16 * bound + 1e-6).item(), "sum_j dV identity"
    say(f"max size backward: sum_j dV identity holds, worst {float((err / (U_BF16 * bound)).max()):.3f} of the bound")
    del g, o, lse, dq, dk, dv
    torch.cuda.empty_cache()


def test_large_plan_column_view_built_beside_the_schedule():
    """A causal mask over 196,608 tokens has 1,180,416 tiles: the plan builds its column
    view (read by the dK/dV kernel and both gradient launch orders) on a second thread
    beside the schedule.  Checked: sampled dQ rows against the oracle, the sum_j dV
    identity over every key, and plans built twice give bit-identical gradients."""
    import torch
    s, hq, hkv, d = 196_608, 1, 1, 64
    scale = 1.0 / np.sqrt(d)
    rng = np.random.default_rng(97)
    qb, kb, vb = W.random_inputs(rng, s, s, hq, hkv, d)
    gb = W.random_grad(rng, s, hq, d)
    slices = [(0, s, 0, s, 1)]
    plan = api.Plan.from_slices(slices, s, s, hq, hkv, d)
    assert plan.info()["nnz"] >= 1 << 20
    plan.upload()
    q, k, v, g = (api.to_device_bf16(x) for x in (qb, kb, vb, gb))
    say(f"large plan: S={s} nnz={plan.info()['nnz']}: forward + backward")
    o, lse = api.attn_fwd(q, k, v, plan, scale)
    dq, dk, dv = api.attn_bwd(q, k, v, g, lse, plan, scale)
    again = api.Plan.from_slices(slices, s, s, hq, hkv, d).upload()
    dq2, dk2, dv2 = api.attn_bwd(q, k, v, g, lse, again, scale)
    torch.cuda.synchronize()
    for name, a, b in (("dQ", dq, dq2), ("dK", dk, dk2), ("dV", dv, dv2)):
        assert torch.isfinite(a).all().item(), f"non-finite {name}"
        assert torch.equal(a, b), f"{name} differs between two builds of the plan"
    rows = [(0, i) for i in (0, 1, 127, 128, 4095, 65_536, 131_071, s // 2 + 17, s - 2, s - 1)]
    rq, _, _ = oracle.attn_bwd_sampled(qb, kb, vb, gb, slices, scale, rows=rows)
    gq = dq[[i for _, i in rows], 0].cpu().numpy()
    err = float(np.max(np.abs(gq - rq)))
    mag = float(np.max(np.abs(rq)))
    say(f"large plan: sampled max|ddQ| = {err:.3e} (max|ref| {mag:.2e})")
    assert err <= GRAD_TOL * max(1.0, mag)
    lhs = torch.sum(dv, dim=0, dtype=torch.float64)[0]
    rhs = torch.sum(g, dim=(0, 1), dtype=torch.float64)
    bound = torch.sum(g.abs(), dim=(0, 1), dtype=torch.float64)
    assert torch.all((lhs - rhs).abs() <= U_BF16 * bound + 1e-6).item(), "sum_j dV identity"
    plan.close()
    again.close()
    del q, k, v, g, o, lse, dq, dk, dv, dq2, dk2, dv2
    torch.cuda.empty_cache()
