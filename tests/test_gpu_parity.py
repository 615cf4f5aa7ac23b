"""GPU parity of the forward and merge kernels against the fp64 oracle, called through
the C-ABI library.  Tolerances: max|dO| <= 1e-2, max|dLSE| <= 1e-3."""
import numpy as np
import pytest

import oracle
from block_sparse_flash_csr_amd import api
from block_sparse_flash_csr_amd import workloads as W

from gpu_helpers import bf16_floor, compare, dev_bf16, host_bits, say, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    api.library()
    yield
    torch.cuda.synchronize()


def run_fwd(qb, kb, vb, slices, scale, sq, sk, hq, hkv, d, bk=128, plan=None):
    import torch
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    own = plan is None
    if own:
        plan = api.Plan.from_slices(slices, sq, sk, hq, hkv, d, bk=bk).upload()
    o, lse = api.attn_fwd(q, k, v, plan, scale)
    torch.cuda.synchronize()
    out = W.bf16_to_f32(host_bits(o)), lse.cpu().numpy()
    if own:
        plan.close()
    return out


def full_check(qb, kb, vb, slices, scale, what, bk=128):
    sq, hq, d = qb.shape
    sk, hkv, _ = kb.shape
    say(f"{what}: sq={sq} sk={sk} hq={hq} hkv={hkv} d={d} slices={len(slices)} bk={bk}")
    o, lse = run_fwd(qb, kb, vb, slices, scale, sq, sk, hq, hkv, d, bk=bk)
    o_ref, lse_ref = oracle.attn_fwd(qb, kb, vb, slices, scale)
    # O is [sq, hq, d], LSE [hq, sq]: compare with LSE laid out as O's leading axes
    return compare(o, lse.T, o_ref, lse_ref.T, what)


# ---------------------------------------------------------------------------
# element-by-element at sizes the oracle finishes in seconds
# ---------------------------------------------------------------------------
def test_causal_s256_full():
    w = W.causal_s256()
    full_check(w.q, w.k, w.v, w.slices, w.scale, "causal S=256 d=64")


@pytest.mark.parametrize("seed,sq,sk,hq,hkv,d,n", [
    (1, 300, 300, 2, 2, 128, 4),
    (2, 517, 389, 4, 2, 128, 6),
    (3, 640, 640, 2, 1, 64, 3),
    (4, 129, 700, 2, 2, 128, 8),
    (5, 700, 129, 3, 3, 64, 5),
    (6, 1, 50, 1, 1, 128, 2),
])
def test_random_masks_full(seed, sq, sk, hq, hkv, d, n):
    rng = np.random.default_rng(seed)
    slices = W.random_slices(rng, sq, sk, n)
    qb, kb, vb = W.random_inputs(rng, sq, sk, hq, hkv, d)
    full_check(qb, kb, vb, slices, 1.0 / np.sqrt(d), f"random seed={seed}")


def test_every_partial_offset():
    """Causal slices whose diagonal enters the tile at every offset 0..127 and ragged tails."""
    sq, sk, d = 400, 400, 128
    rng = np.random.default_rng(77)
    qb, kb, vb = W.random_inputs(rng, sq, sk, 2, 1, d)
    slices = [(0, sq, 0, sk - 61, 1), (3, 131, 200, 333, 1), (150, 151, 0, 400, 0)]
    full_check(qb, kb, vb, slices, 1.0 / np.sqrt(d), "partial offsets")
    slices = [(q0, q0 + 1, 0, min(sk, q0 + 1 + (q0 % 7)), 0) for q0 in range(0, sq)]
    full_check(qb, kb, vb, slices, 1.0 / np.sqrt(d), "per-row ragged windows")


def test_bk64_plan():
    rng = np.random.default_rng(5)
    sq = sk = 333
    slices = W.random_slices(rng, sq, sk, 5)
    qb, kb, vb = W.random_inputs(rng, sq, sk, 2, 2, 128)
    full_check(qb, kb, vb, slices, 1.0 / np.sqrt(128), "plan bk=64", bk=64)


def _large_logit_inputs(d):
    rng = np.random.default_rng(9)
    sq = sk = 512
    qf = rng.standard_normal((sq, 2, d), dtype=np.float32) * 8.0
    qb = W.bf16_bits(qf)
    _, kb, vb = W.random_inputs(rng, sq, sk, 2, 2, d)
    return qb, kb, vb


@pytest.mark.parametrize("d", [128, 64])
def test_large_logits_exercise_rescale(d):
    """Tile maxima that jump by more than the rescale threshold (at d = 64 the weights
    are checked after the fact, so these steps take the recomputation path)."""
    qb, kb, vb = _large_logit_inputs(d)
    sq = sk = qb.shape[0]
    if d == 128:
        full_check(qb, kb, vb, [(0, sq, 0, sk, 1)], 1.0 / np.sqrt(d), f"Q x8 causal d={d}")
    # increasing scores along keys: the max moves on every tile
    kf = W.bf16_to_f32(kb).copy()
    kf += np.linspace(0, 6, sk, dtype=np.float32)[:, None, None] * np.sign(
        W.bf16_to_f32(qb).mean(axis=0, keepdims=True))
    full_check(qb, W.bf16_bits(kf), vb, [(0, sq, 0, sk, 0)], 1.0 / np.sqrt(d),
               f"growing max full d={d}")
    # scores that grow by tens of log2 units within one tile: the first weights taken
    # against the running max overflow to infinity and must be recomputed
    kf2 = W.bf16_to_f32(kb).copy()
    kf2 += np.linspace(0, 40, sk, dtype=np.float32)[:, None, None] * np.sign(
        W.bf16_to_f32(qb).mean(axis=0, keepdims=True))
    full_check(qb, W.bf16_bits(kf2), vb, [(0, sq, 0, sk, 0)], 1.0 / np.sqrt(d),
               f"steep max full d={d}")


@pytest.mark.parametrize("d", [128, 64])
def test_rescale_threshold_zero_equals_default(d):
    """The conditional rescale changes only rounding: with tau = 0 (the max moves whenever
    it grows) and the default tau = 8 the outputs both meet the oracle's tolerance and
    agree with each other to a few bf16 units."""
    import torch
    rng = np.random.default_rng(90 + d)
    sq, sk = 600, 700
    slices = W.random_slices(rng, sq, sk, 5) + [(0, sq, 0, sk, 1)]
    qb, kb, vb = W.random_inputs(rng, sq, sk, 3, 1, d)
    kf = W.bf16_to_f32(kb).copy()      # maxima that grow along the keys
    kf += np.linspace(0, 10, sk, dtype=np.float32)[:, None, None] * np.sign(
        W.bf16_to_f32(qb).mean(axis=0, keepdims=True)[:, :1])
    kb = W.bf16_bits(kf)
    o_ref, lse_ref = oracle.attn_fwd(qb, kb, vb, slices, 1.0 / np.sqrt(d))
    outs = {}
    try:
        for tau in (0.0, 8.0):
            api.set_rescale_threshold(tau)
            o, lse = run_fwd(qb, kb, vb, slices, 1.0 / np.sqrt(d), sq, sk, 3, 1, d)
            compare(o, lse.T, o_ref, lse_ref.T, f"tau={tau} d={d}")
            outs[tau] = (o, lse)
    finally:
        api.set_rescale_threshold(8.0)
    assert float(np.max(np.abs(outs[0.0][0] - outs[8.0][0]))) <= 1.6e-2
    fin = np.isfinite(outs[8.0][1])
    assert float(np.max(np.abs(outs[0.0][1][fin] - outs[8.0][1][fin]))) <= 1e-4


class OutputFormatBreach(AssertionError):
    """The 1e-2 bar fails only by the bf16 output format: rounding the exact O to bf16
    alone already exceeds it."""


@pytest.mark.xfail(raises=OutputFormatBreach, strict=False,
                   reason="rows nearly one-hot with |O| >= 4: rounding the exact output to bf16 alone "
                          "gives 0.0129 > 1e-2")
def test_one_hot_rows_d64():
    """Q x8 causal at d = 64: some rows are nearly one-hot with |O| in [4, 8), where bf16
    output rounding alone reaches 0.0156.  The kernel's error must be that rounding plus
    at most the bf16 weights' share (2^-9 of |O|); the 1e-2 bar itself is a known breach."""
    d = 64
    qb, kb, vb = _large_logit_inputs(d)
    sq = sk = qb.shape[0]
    sl = [(0, sq, 0, sk, 1)]
    say("Q x8 causal d=64 (nearly one-hot rows)")
    o, lse = run_fwd(qb, kb, vb, sl, 1.0 / np.sqrt(d), sq, sk, 2, 2, d)
    o_ref, lse_ref = oracle.attn_fwd(qb, kb, vb, sl, 1.0 / np.sqrt(d))
    floor = bf16_floor(o_ref)
    err = float(np.max(np.abs(o.astype(np.float64) - o_ref)))
    dl = float(np.max(np.abs(lse.T - lse_ref.T)))
    say(f"Q x8 causal d=64: max|dO| {err:.3e} (bf16 output floor {floor:.3e}), max|dLSE| {dl:.3e}")
    assert not np.isnan(o).any() and dl <= 1e-3
    assert err <= floor + 2.0 ** -9 * float(np.max(np.abs(o_ref))), (err, floor)
    if err > 1e-2:
        raise OutputFormatBreach(f"max|dO| {err} > 1e-2 with a bf16 output floor of {floor}")


def test_fully_masked_rows_and_empty_tiles():
    sq, sk, d = 384, 256, 128
    rng = np.random.default_rng(10)
    qb, kb, vb = W.random_inputs(rng, sq, sk, 2, 2, d)
    # rows 128..255 have no key at all; rows 300..383 only via a rectangular causal slice
    slices = [(0, 128, 0, 256, 1), (256, 384, 100, 140, 1)]
    full_check(qb, kb, vb, slices, 0.1, "masked rows")
    full_check(qb, kb, vb, [], 0.1, "empty mask")


def test_deterministic_and_masked_perturbation_invisible():
    import torch
    sq = sk = 384
    d = 128
    rng = np.random.default_rng(12)
    qb, kb, vb = W.random_inputs(rng, sq, sk, 2, 1, d)
    slices = [(0, 200, 0, 200, 1), (200, 384, 64, 300, 0)]
    say("determinism + masked perturbation")
    o1, l1 = run_fwd(qb, kb, vb, slices, 0.1, sq, sk, 2, 1, d)
    o2, l2 = run_fwd(qb, kb, vb, slices, 0.1, sq, sk, 2, 1, d)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # keys >= 300 are masked for every row; keys 200..299 for rows < 200
    big = W.bf16_bits(np.array([3.0e4], np.float32))[0]
    kb2, vb2 = kb.copy(), vb.copy()
    kb2[300:] = big
    vb2[300:] = big
    kb2[200:300, :, 1::3] = big
    vb2[200:300] = big
    o3, l3 = run_fwd(qb, kb2, vb2, slices, 0.1, sq, sk, 2, 1, d)
    assert np.array_equal(o1[:200], o3[:200]) and np.array_equal(l1[:, :200], l3[:, :200])
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# full sizes, sampled rows, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------
def sampled_check(w, plan, rows, what):
    import torch
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    say(f"{what}: launching forward")
    o, lse = api.attn_fwd(q, k, v, plan, w.scale)
    torch.cuda.synchronize()
    assert not torch.isnan(o.float()).any().item(), "NaN in O"
    r = np.array(rows, np.int64)
    hs = torch.from_numpy(r[:, 0]).cuda()
    is_ = torch.from_numpy(r[:, 1]).cuda()
    o_s = W.bf16_to_f32(host_bits(o[is_, hs]))
    l_s = lse[hs, is_].cpu().numpy()
    o_ref, lse_ref = oracle.attn_fwd(w.q, w.k, w.v, w.slices, w.scale, rows=rows)
    compare(o_s, l_s, o_ref, lse_ref, what)
    return o, lse


def workload_full_check(w, what):
    """Every (head, row) output of a full-size workload, on the plan the benchmark times."""
    import torch
    plan = api.plan_from_workload(w)
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    say(f"{what}: launching forward ({w.sq} rows x {w.hq} heads)")
    o, lse = api.attn_fwd(q, k, v, plan, w.scale)
    torch.cuda.synchronize()
    o_gpu, l_gpu = W.bf16_to_f32(host_bits(o)), lse.cpu().numpy()
    plan.close()
    say(f"{what}: oracle on every row")
    o_ref, lse_ref = oracle.attn_fwd(w.q, w.k, w.v, w.slices, w.scale)
    compare(o_gpu, l_gpu.T, o_ref, lse_ref.T, what)


def test_varlen_causal_t16384_full():
    workload_full_check(W.varlen_causal_t16384(), "varlen causal t16384, every output")


def test_block_sparse_strided_s32768_full():
    workload_full_check(W.block_sparse_strided_s32768(), "block-sparse strided s32768, every output")


def test_range_slices_s65536_sampled():
    w = W.range_slices_s65536()
    plan = api.plan_from_workload(w)
    extra = [s[0] for s in w.slices[16:40]] + [s[1] - 1 for s in w.slices[16:40]]
    sampled_check(w, plan, sample_rows(w, 256, 4, extra), "range slices s65536 GQA")


@pytest.mark.parametrize("q_chunk", [7, 3])
def test_kv_split_q8192_split_merge_sampled(q_chunk):
    import torch
    w = W.kv_split_q8192(q_chunk=q_chunk)
    c, nc = w.extra["chunk"], w.extra["n_chunks"]
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    plans = [api.Plan.from_slices(sl, c, c, w.hq, w.hkv, w.d).upload()
             for sl in w.extra["chunk_slices"]]
    say(f"kv split q8192 q_chunk={q_chunk}: 8 partial forwards + merge")
    parts = [api.attn_fwd(q, k[t * c:(t + 1) * c], v[t * c:(t + 1) * c], plans[t], w.scale)
             for t in range(nc)]
    o, lse = api.attn_merge([p[0] for p in parts], [p[1] for p in parts])
    torch.cuda.synchronize()
    rows = sample_rows(w, 192, 5)
    r = np.array(rows, np.int64)
    hs = torch.from_numpy(r[:, 0]).cuda()
    is_ = torch.from_numpy(r[:, 1]).cuda()
    o_s = W.bf16_to_f32(host_bits(o[is_, hs]))
    l_s = lse[hs, is_].cpu().numpy()
    o_ref, lse_ref = oracle.attn_fwd(w.q, w.k, w.v, w.slices, w.scale, rows=rows)
    compare(o_s, l_s, o_ref, lse_ref, f"kv split q8192 split+merge q_chunk={q_chunk}")
    for p in plans:
        p.close()


# ---------------------------------------------------------------------------
# merge kernel on synthetic partials
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,t,h,d", [(1, 77, 3, 128), (3, 300, 4, 64), (8, 1000, 5, 128),
                                     (16, 129, 2, 128)])
def test_merge_synthetic(n, t, h, d):
    import torch
    rng = np.random.default_rng(n * 1000 + t)
    # partial outputs: averages of value rows, so std ~0.5; LSEs spread over a few units
    o_bits = W.bf16_bits(0.5 * rng.standard_normal((n, t, h, d), dtype=np.float32))
    lse_p = (3.0 * rng.standard_normal((n, h, t))).astype(np.float32)
    lse_p[rng.random((n, h, t)) < 0.2] = -np.inf
    lse_p[:, 0, :5] = -np.inf          # rows where every partial is empty
    say(f"merge n={n} t={t} h={h} d={d}")
    parts = [dev_bf16(o_bits[i]) for i in range(n)]
    lses = [torch.from_numpy(lse_p[i]).cuda() for i in range(n)]
    o, lse = api.attn_merge(parts, lses)
    torch.cuda.synchronize()
    o_f = W.bf16_to_f32(o_bits).astype(np.float64)          # [n, t, h, d]
    po = o_f.transpose(0, 2, 1, 3).reshape(n, h * t, d)
    pl = lse_p.reshape(n, h * t).astype(np.float64)
    om, lm = oracle.merge(po, pl)
    o_gpu = W.bf16_to_f32(host_bits(o)).transpose(1, 0, 2).reshape(h * t, d)
    compare(o_gpu, lse.cpu().numpy().reshape(h * t), om, lm, f"merge n={n}")


# ---------------------------------------------------------------------------
# plan churn: device metadata buffers are pooled and reused without waiting
# ---------------------------------------------------------------------------
def test_plan_churn_reuses_buffers_safely():
    """Plans of two different masks are built, uploaded, launched and destroyed back to
    back with no synchronisation, some of them launched on a second stream; every
    output must equal (bitwise) the output of a plan that lived alone."""
    import torch
    sq = sk = 640
    d = 128
    rng = np.random.default_rng(21)
    qb, kb, vb = W.random_inputs(rng, sq, sk, 2, 2, d)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    masks = [[(0, sq, 0, sk, 1)], W.random_slices(rng, sq, sk, 9)]
    say("plan churn: references")
    ref = []
    for m in masks:
        p = api.Plan.from_slices(m, sq, sk, 2, 2, d).upload()
        o, l = api.attn_fwd(q, k, v, p, 0.09)
        torch.cuda.synchronize()
        ref.append((o.clone(), l.clone()))
        p.close()
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    outs = []
    say("plan churn: 24 plans without synchronisation")
    for i in range(24):
        m = i % 2
        p = api.Plan.from_slices(masks[m], sq, sk, 2, 2, d).upload(main)
        o = torch.empty((sq, 2, d), dtype=torch.bfloat16, device="cuda")
        l = torch.empty((2, sq), dtype=torch.float32, device="cuda")
        if i % 3 == 2:
            side.wait_stream(main)
            api.attn_fwd(q, k, v, p, 0.09, out=o, lse=l, stream=side)
            main.wait_stream(side)
        else:
            api.attn_fwd(q, k, v, p, 0.09, out=o, lse=l, stream=main)
        p.close()
        outs.append((m, o, l))
    torch.cuda.synchronize()
    for i, (m, o, l) in enumerate(outs):
        assert torch.equal(o, ref[m][0]) and torch.equal(l, ref[m][1]), f"plan {i} (mask {m}) differs"


def test_plans_uploaded_ahead_and_launched_on_any_stream():
    """Each plan is uploaded one iteration before its launch (the benchmark's pipeline)
    and launched on a stream the caller never ordered after the upload: every launch is
    ordered after its plan's copy by the library itself."""
    import torch
    sq = sk = 512
    d = 128
    rng = np.random.default_rng(23)
    qb, kb, vb = W.random_inputs(rng, sq, sk, 2, 2, d)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    masks = [[(0, sq, 0, sk, 1)], W.random_slices(rng, sq, sk, 7), W.random_slices(rng, sq, sk, 3)]
    ref = []
    for m in masks:
        p = api.Plan.from_slices(m, sq, sk, 2, 2, d).upload()
        o, l = api.attn_fwd(q, k, v, p, 0.09)
        torch.cuda.synchronize()
        ref.append((o.clone(), l.clone()))
        p.close()
    n = 30
    outs = [(torch.empty((sq, 2, d), dtype=torch.bfloat16, device="cuda"),
             torch.empty((2, sq), dtype=torch.float32, device="cuda")) for _ in range(n)]
    up = torch.cuda.Stream()
    runs = [torch.cuda.current_stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    say(f"plans uploaded ahead: {n} launches over two streams, uploads on a third")
    nxt = api.Plan.from_slices(masks[0], sq, sk, 2, 2, d).upload(up)
    for i in range(n):
        cur = nxt
        nxt = api.Plan.from_slices(masks[(i + 1) % 3], sq, sk, 2, 2, d).upload(up)
        api.attn_fwd(q, k, v, cur, 0.09, out=outs[i][0], lse=outs[i][1], stream=runs[i % 2])
        cur.close()
    nxt.close()
    torch.cuda.synchronize()
    for i, (o, l) in enumerate(outs):
        assert torch.equal(o, ref[i % 3][0]) and torch.equal(l, ref[i % 3][1]), f"launch {i} differs"


# ---------------------------------------------------------------------------
# rows split into parts inside one call (partials merged by a second kernel)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed,sq,sk,hq,hkv,d,kind", [
    (31, 256, 12000, 2, 1, 128, "full"),
    (32, 200, 9000, 2, 2, 64, "causal"),
    (33, 130, 20000, 1, 1, 128, "gappy"),
])
def test_split_rows_full(seed, sq, sk, hq, hkv, d, kind):
    rng = np.random.default_rng(seed)
    if kind == "full":
        slices = [(0, sq, 0, sk, 0)]
    elif kind == "causal":
        slices = [(0, sq, 0, sk, 1)]
    else:
        # rows 0..64 see only early keys, 70..129 only late keys (causal), 65..69 none:
        # some parts hold no key of a row, and some rows have no key at all
        slices = [(0, 65, 0, 3000, 0), (70, 130, 15000, sk, 1)]
    qb, kb, vb = W.random_inputs(rng, sq, sk, hq, hkv, d)
    plan = api.Plan.from_slices(slices, sq, sk, hq, hkv, d)
    inf = plan.info()
    assert inf["n_splits"] > 0, inf
    say(f"split rows {kind}: units={inf['n_units']} splits={inf['n_splits']}")
    plan.close()
    full_check(qb, kb, vb, slices, 1.0 / np.sqrt(d), f"split rows {kind}")


def test_split_plan_shared_by_two_streams_at_once():
    """One plan with split rows launched on two streams with no ordering between them,
    each launch with its own workspace: the plan holds no per-launch state, so both
    outputs equal the oracle's (and each other, bit for bit)."""
    import torch
    sq, sk, hq, hkv, d = 256, 12000, 2, 1, 128
    rng = np.random.default_rng(37)
    slices = [(0, sq, 0, sk, 1), (0, 40, 5000, 5100, 0)]
    qb, kb, vb = W.random_inputs(rng, sq, sk, hq, hkv, d)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    plan = api.Plan.from_slices(slices, sq, sk, hq, hkv, d).upload()
    inf = plan.info()
    assert inf["n_splits"] > 0 and inf["workspace_bytes"] > 0, inf
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [api.workspace_for(plan) for _ in streams]
    outs = [[(torch.empty((sq, hq, d), dtype=torch.bfloat16, device="cuda"),
              torch.empty((hq, sq), dtype=torch.float32, device="cuda")) for _ in range(6)] for _ in streams]
    torch.cuda.synchronize()
    say(f"split plan on two streams at once: units={inf['n_units']} splits={inf['n_splits']}")
    for i in range(6):
        for s_i, s in enumerate(streams):
            o, l = outs[s_i][i]
            api.attn_fwd(q, k, v, plan, 1.0 / np.sqrt(d), out=o, lse=l, workspace=wss[s_i], stream=s)
    torch.cuda.synchronize()
    plan.close()
    o_ref, lse_ref = oracle.attn_fwd(qb, kb, vb, slices, 1.0 / np.sqrt(d))
    o0, l0 = outs[0][0]
    compare(W.bf16_to_f32(host_bits(o0)), l0.cpu().numpy().T, o_ref, lse_ref.T, "split plan, two streams")
    for s_i in range(2):
        for i in range(6):
            o, l = outs[s_i][i]
            assert torch.equal(o, o0) and torch.equal(l, l0), (s_i, i)


def test_one_token_tensors_need_a_full_row_stride():
    """A tensor with a single token still needs stride_tok >= d (the kernels size their
    buffer ranges as rows x stride): a smaller stride is refused, not read short."""
    import ctypes
    import torch
    d = 128
    plan = api.Plan.from_slices([(0, 1, 0, 50, 0)], 1, 50, 2, 1, d).upload()
    lib = api.library()
    q = torch.zeros((1, 2, d), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((50, 1, d), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros((1, 2, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((2, 1), dtype=torch.float32, device="cuda")
    tq_bad = api.Tensor(ctypes.c_void_p(q.data_ptr()), 8, d)
    tq = api.Tensor(ctypes.c_void_p(q.data_ptr()), 2 * d, d)
    tkv = api.Tensor(ctypes.c_void_p(kv.data_ptr()), d, d)
    to = api.Tensor(ctypes.c_void_p(o.data_ptr()), 2 * d, d)

    def call(tq_, to_):
        return lib.bsfa_attn_fwd(ctypes.byref(tq_), ctypes.byref(tkv), ctypes.byref(tkv), plan.handle, 0.1,
                                 ctypes.byref(to_), ctypes.c_void_p(lse.data_ptr()), 1, None, 0,
                                 api._stream_handle())

    assert call(tq_bad, to) == 2
    assert call(tq, api.Tensor(ctypes.c_void_p(o.data_ptr()), 0, d)) == 2
    assert call(tq, to) == 0
    torch.cuda.synchronize()
    plan.close()


def test_plans_from_several_host_threads():
    """Four host threads build, upload, launch and destroy plans at the same time, each on
    its own stream (the plan pools, the staging images and the copy ordering are shared
    by all of them); every output equals the single-threaded reference bit for bit."""
    import threading
    import torch
    sq = sk = 384
    d = 128
    rng = np.random.default_rng(29)
    qb, kb, vb = W.random_inputs(rng, sq, sk, 2, 2, d)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    masks = [[(0, sq, 0, sk, 1)], W.random_slices(rng, sq, sk, 5), W.random_slices(rng, sq, sk, 9)]
    ref = []
    for m in masks:
        p = api.Plan.from_slices(m, sq, sk, 2, 2, d).upload()
        o, l = api.attn_fwd(q, k, v, p, 0.09)
        torch.cuda.synchronize()
        ref.append((o.clone(), l.clone()))
        p.close()
    n_threads, n_iter = 4, 12
    outs = [[(torch.empty((sq, 2, d), dtype=torch.bfloat16, device="cuda"),
              torch.empty((2, sq), dtype=torch.float32, device="cuda")) for _ in range(n_iter)]
            for _ in range(n_threads)]
    streams = [torch.cuda.Stream() for _ in range(n_threads)]
    torch.cuda.synchronize()
    errors = []

    def worker(t):
        try:
            torch.cuda.set_device(0)
            s = streams[t]
            for i in range(n_iter):
                m = (t + i) % 3
                p = api.Plan.from_slices(masks[m], sq, sk, 2, 2, d).upload(s)
                api.attn_fwd(q, k, v, p, 0.09, out=outs[t][i][0], lse=outs[t][i][1], stream=s)
                p.close()
        except Exception as e:   # reported below, in the test's own thread
            errors.append(repr(e))

    say(f"plans from {n_threads} host threads x {n_iter}")
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(n_threads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(n_threads):
        for i in range(n_iter):
            m = (t + i) % 3
            assert torch.equal(outs[t][i][0], ref[m][0]) and torch.equal(outs[t][i][1], ref[m][1]), (t, i)


@pytest.mark.parametrize("bk", [192, 256])
def test_wide_key_tile_plans(bk):
    """Plans with key tiles of 192 and 256 keys (3 and 4 kernel steps per CSR entry)."""
    rng = np.random.default_rng(bk)
    sq, sk = 517, 1100
    slices = W.random_slices(rng, sq, sk, 6) + [(0, sq, 0, sk, 1)]
    qb, kb, vb = W.random_inputs(rng, sq, sk, 4, 2, 128)
    full_check(qb, kb, vb, slices, 1.0 / np.sqrt(128), f"plan bk={bk}", bk=bk)


def test_zero_length_extents():
    """No keys at all (every row gets O = 0, LSE = -inf) and no queries (nothing to do)."""
    import torch
    d = 128
    rng = np.random.default_rng(61)
    qb, _, _ = W.random_inputs(rng, 100, 1, 2, 1, d)
    q = dev_bf16(qb)
    k = torch.empty((0, 1, d), dtype=torch.bfloat16, device="cuda")
    plan = api.Plan.from_slices([], 100, 0, 2, 1, d).upload()
    o = torch.full((100, 2, d), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((2, 100), dtype=torch.float32, device="cuda")
    api.attn_fwd(q, k, k, plan, 0.1, out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool((o.float() == 0).all()) and bool(torch.isneginf(lse).all())
    plan.close()
    q0 = torch.empty((0, 2, d), dtype=torch.bfloat16, device="cuda")
    kv = dev_bf16(W.random_inputs(rng, 1, 50, 2, 1, d)[1])
    plan = api.Plan.from_slices([], 0, 50, 2, 1, d).upload()
    o0, l0 = api.attn_fwd(q0, kv, kv, plan, 0.1)
    torch.cuda.synchronize()
    assert o0.numel() == 0
    # backward without queries: every key's gradient is zero
    dq, dk, dv = api.attn_bwd(q0, kv, kv, q0, l0, plan, 0.1)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and bool((dk == 0).all()) and bool((dv == 0).all())
    plan.close()
    # backward without keys: dQ is zero
    plan = api.Plan.from_slices([], 100, 0, 2, 1, d).upload()
    g = dev_bf16(W.random_grad(rng, 100, 2, d))
    dq, dk, dv = api.attn_bwd(q, k, k, g, lse, plan, 0.1)
    torch.cuda.synchronize()
    assert bool((dq == 0).all()) and dk.numel() == 0 and dv.numel() == 0
    plan.close()
    # merge of empty partials
    e = torch.empty((0, 2, d), dtype=torch.bfloat16, device="cuda")
    le = torch.empty((2, 0), dtype=torch.float32, device="cuda")
    om, lm = api.attn_merge([e, e], [le, le])
    assert om.numel() == 0 and lm.numel() == 0


def test_block_code_plan_with_ragged_blocks():
    """A plan from a block code map (blocks of 48 x 40, clipped at ragged extents, codes
    empty / full / causal drawn at random) against the oracle on the equivalent slices."""
    import torch
    sq, sk, hq, hkv, d = 517, 389, 4, 2, 128
    rng = np.random.default_rng(47)
    nbq, nbk = -(-sq // 48), -(-sk // 40)
    codes = rng.integers(0, 3, size=(nbq, nbk)).astype(np.uint8)
    qb, kb, vb = W.random_inputs(rng, sq, sk, hq, hkv, d)
    plan = api.Plan.from_blocks(codes, 48, 40, sq, sk, hq, hkv, d).upload()
    say(f"block code plan: {nbq} x {nbk} blocks of 48 x 40, sq={sq} sk={sk}")
    o, lse = api.attn_fwd(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), plan, 0.1)
    torch.cuda.synchronize()
    plan.close()
    o_ref, lse_ref = oracle.attn_fwd(qb, kb, vb, W.block_slices(codes, 48, 40, sq, sk), 0.1)
    compare(W.bf16_to_f32(host_bits(o)), lse.cpu().numpy().T, o_ref, lse_ref.T, "block code plan")


@pytest.mark.parametrize("causal", [True, False])
def test_varlen_plans_with_empty_and_tiny_documents(causal):
    """Varlen plans, causal and full within documents, including an empty document and
    one-token documents, against the oracle on the equivalent slices."""
    import torch
    lengths = [0, 1, 130, 1, 257, 0, 64, 300]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    s, hq, hkv, d = int(cu[-1]), 4, 2, 128
    rng = np.random.default_rng(53 + causal)
    qb, kb, vb = W.random_inputs(rng, s, s, hq, hkv, d)
    plan = api.Plan.from_varlen(cu, hq, hkv, d, causal=causal).upload()
    say(f"varlen plan causal={causal}: documents {lengths}")
    o, lse = api.attn_fwd(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), plan, 0.1)
    torch.cuda.synchronize()
    plan.close()
    slices = [(int(cu[t]), int(cu[t + 1]), int(cu[t]), int(cu[t + 1]), 1 if causal else 0)
              for t in range(len(lengths)) if lengths[t] > 0]
    o_ref, lse_ref = oracle.attn_fwd(qb, kb, vb, slices, 0.1)
    compare(W.bf16_to_f32(host_bits(o)), lse.cpu().numpy().T, o_ref, lse_ref.T, f"varlen causal={causal}")


def test_plan_churn_over_many_sizes():
    """Plans of very different sizes (so pooled staging images and device buffers of
    several capacities are taken, outgrown and reused) built, launched and destroyed
    back to back on two streams with no synchronisation; every output equals the output
    of the same plan run alone."""
    import torch
    rng = np.random.default_rng(67)
    shapes = [(int(rng.integers(1, 4500)), int(rng.integers(1, 4500))) for _ in range(8)]
    cases = []
    for sq, sk in shapes:
        sl = W.random_slices(rng, sq, sk, int(rng.integers(1, 9))) + [(0, sq, 0, sk, int(rng.integers(0, 2)))]
        qb, kb, vb = W.random_inputs(rng, sq, sk, 2, 1, 128)
        q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
        p = api.Plan.from_slices(sl, sq, sk, 2, 1, 128).upload()
        o, l = api.attn_fwd(q, k, v, p, 0.1)
        torch.cuda.synchronize()
        p.close()
        cases.append((sl, sq, sk, q, k, v, o.clone(), l.clone()))
    streams = [torch.cuda.current_stream(), torch.cuda.Stream()]
    order = [int(x) for x in rng.integers(0, len(cases), 40)]
    outs = []
    say(f"plan churn over sizes {shapes}: 40 launches")
    for n, c in enumerate(order):
        sl, sq, sk, q, k, v, _, _ = cases[c]
        s = streams[n % 2]
        o = torch.empty((sq, 2, 128), dtype=torch.bfloat16, device="cuda")
        l = torch.empty((2, sq), dtype=torch.float32, device="cuda")
        s.wait_stream(torch.cuda.current_stream())   # the outputs were allocated on the current stream
        p = api.Plan.from_slices(sl, sq, sk, 2, 1, 128).upload(s)
        api.attn_fwd(q, k, v, p, 0.1, out=o, lse=l, stream=s)
        p.close()
        outs.append((c, o, l))
    torch.cuda.synchronize()
    for n, (c, o, l) in enumerate(outs):
        assert torch.equal(o, cases[c][6]) and torch.equal(l, cases[c][7]), f"launch {n} (case {c}) differs"
