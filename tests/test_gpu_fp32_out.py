"""fp32 outputs of the forward and the merge (the typed entry points) against the fp64
oracle, and against the bf16 path.

An fp32 O is the normalised fp32 value whose round-to-nearest-even the bf16 path stores,
so the two calls must agree bit for bit after rounding, LSE included, on every kind of
plan (full-size workloads, d = 64, split rows).  Without the bf16 output's rounding the
forward meets the 1e-2 bar also where the bf16 output cannot (rows of a few keys with
|O| >= 2: the sweep's seeds 6 and 13 and the nearly one-hot d = 64 rows), and KV-split
partials kept in fp32 merge to the unsplit result (UltraAttn blog 3.2)."""
import numpy as np
import pytest

import oracle
from block_sparse_flash_csr_amd import api
from block_sparse_flash_csr_amd import workloads as W

from gpu_helpers import compare, dev_bf16, host_bits, sample_rows, say
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


def both_outputs(q, k, v, plan, scale):
    """(O bf16, LSE) and (O fp32, LSE) of one plan."""
    import torch
    o16, l16 = api.attn_fwd(q, k, v, plan, scale)
    o32, l32 = api.attn_fwd(q, k, v, plan, scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert o32.dtype == torch.float32
    return o16, l16, o32, l32


def assert_rounds_to(o16, l16, o32, l32, what):
    import torch
    assert not torch.isnan(o32).any(), f"{what}: NaN in fp32 O"
    r = o32.to(torch.bfloat16)           # round to nearest even
    same = torch.equal(r.view(torch.int16), o16.view(torch.int16))
    n_diff = int((r.view(torch.int16) != o16.view(torch.int16)).sum())
    say(f"{what}: bf16(O fp32) == O bf16 bitwise: {same} ({n_diff} elements differ); "
        f"LSE equal: {torch.equal(l16, l32)}")
    assert same, f"{what}: {n_diff} elements of bf16(O fp32) differ from the bf16 output"
    assert torch.equal(l16, l32), f"{what}: LSE differs between the two output types"


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_fp32_output_rounds_to_the_bf16_output_workloads(cfg):
    w = W.WORKLOADS[cfg]()
    say(f"fp32 vs bf16 O: {w.name}")
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    plan = api.Plan.from_slices(w.slices, w.sq, w.sk, w.hq, w.hkv, w.d).upload()
    assert_rounds_to(*both_outputs(q, k, v, plan, w.scale), w.name)
    plan.close()


@pytest.mark.parametrize("kind", ["split_rows", "gqa_ragged_d64", "bk64"])
def test_fp32_output_rounds_to_the_bf16_output_plans(kind):
    rng = np.random.default_rng(51)
    if kind == "split_rows":
        sq, sk, hq, hkv, d, bk = 256, 12000, 2, 1, 128, 128
        slices = [(0, sq, 0, sk, 1), (0, 40, 5000, 5100, 0)]
    elif kind == "gqa_ragged_d64":
        sq, sk, hq, hkv, d, bk = 333, 517, 6, 2, 64, 128
        slices = W.random_slices(rng, sq, sk, 7)
    else:
        sq, sk, hq, hkv, d, bk = 300, 451, 2, 2, 128, 64
        slices = [(0, sq, 0, sk, 1), (10, 90, 200, 450, 0)]
    qb, kb, vb = W.random_inputs(rng, sq, sk, hq, hkv, d)
    plan = api.Plan.from_slices(slices, sq, sk, hq, hkv, d, bk=bk).upload()
    if kind == "split_rows":
        assert plan.info()["n_splits"] > 0
    say(f"fp32 vs bf16 O: {kind} sq={sq} sk={sk} hq={hq} hkv={hkv} d={d} bk={bk}")
    o16, l16, o32, l32 = both_outputs(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), plan, 0.11)
    plan.close()
    assert_rounds_to(o16, l16, o32, l32, kind)
    o_ref, lse_ref = oracle.attn_fwd(qb, kb, vb, slices, 0.11)
    compare(o32.cpu().numpy(), l32.cpu().numpy().T, o_ref, lse_ref.T, f"{kind} fp32 O")


@pytest.mark.parametrize("seed", range(256))
def test_fp32_output_sweep_meets_the_bar(seed):
    """The forward sweep's cases and 232 more of its generator, with fp32 O: all of them,
    the two whose bf16 output is a known breach included, meet max|dO| <= 1e-2 and
    max|dLSE| <= 1e-3; the bf16 call's output is that fp32 output rounded to nearest even,
    bit for bit, and its LSE is the same, so a bf16 output that misses the 1e-2 bar misses
    it by its own rounding only (at most half a bf16 step of |O|)."""
    import torch
    _, sq, sk, hq, hkv, d, bk, slices, scale, qb, kb, vb = draw_case(seed)
    what = f"sweep fwd fp32 O seed={seed} sq={sq} sk={sk} hq={hq} hkv={hkv} d={d} bk={bk}"
    say(what)
    plan = api.Plan.from_slices(slices, sq, sk, hq, hkv, d, bk=bk).upload()
    o16, l16, o, lse = both_outputs(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), plan, scale)
    plan.close()
    assert_rounds_to(o16, l16, o, lse, what)
    o_ref, lse_ref = oracle.attn_fwd(qb, kb, vb, slices, scale)
    compare(o.cpu().numpy(), lse.cpu().numpy().T, o_ref, lse_ref.T, what)
    err16 = float(np.max(np.abs(W.bf16_to_f32(host_bits(o16)).astype(np.float64) - o_ref))) if o_ref.size else 0.0
    say(f"{what}: bf16 output max|dO| {err16:.3e}{' (beyond 1e-2 by its rounding)' if err16 > 1e-2 else ''}")


def test_fp32_output_one_hot_rows_d64():
    """Q x8 causal at d = 64 (nearly one-hot rows, |O| in [4, 8)): the bf16 output's
    rounding alone exceeds 1e-2 there; the fp32 output meets the bar."""
    import torch
    d = 64
    rng = np.random.default_rng(9)
    sq = sk = 512
    qb = W.bf16_bits(rng.standard_normal((sq, 2, d), dtype=np.float32) * 8.0)
    _, kb, vb = W.random_inputs(rng, sq, sk, 2, 2, d)
    sl = [(0, sq, 0, sk, 1)]
    say("Q x8 causal d=64, fp32 O")
    plan = api.Plan.from_slices(sl, sq, sk, 2, 2, d).upload()
    o, lse = api.attn_fwd(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), plan, 1.0 / np.sqrt(d),
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    plan.close()
    o_ref, lse_ref = oracle.attn_fwd(qb, kb, vb, sl, 1.0 / np.sqrt(d))
    compare(o.cpu().numpy(), lse.cpu().numpy().T, o_ref, lse_ref.T, "Q x8 causal d=64 fp32 O")


@pytest.mark.parametrize("n,t,h,d", [(1, 77, 3, 128), (3, 300, 4, 64), (8, 1000, 5, 128),
                                     (16, 129, 2, 128)])
def test_merge_fp32_partials_synthetic(n, t, h, d):
    """fp32 partials into fp32 and bf16 results, bf16 partials into an fp32 result, against
    the oracle's merge of the same partial values."""
    import torch
    rng = np.random.default_rng(n * 1000 + t + 7)
    o_p = (0.5 * rng.standard_normal((n, t, h, d))).astype(np.float32)
    lse_p = (3.0 * rng.standard_normal((n, h, t))).astype(np.float32)
    lse_p[rng.random((n, h, t)) < 0.2] = -np.inf
    lse_p[:, 0, :5] = -np.inf          # rows where every partial is empty
    lses = [torch.from_numpy(lse_p[i]).cuda() for i in range(n)]
    pl = lse_p.reshape(n, h * t).astype(np.float64)

    def flat(x):                       # [t, h, d] -> [h * t, d]
        return np.asarray(x, np.float64).transpose(1, 0, 2).reshape(h * t, d)

    say(f"merge fp32 partials n={n} t={t} h={h} d={d}")
    parts32 = [torch.from_numpy(o_p[i]).cuda() for i in range(n)]
    om, lm = oracle.merge(o_p.astype(np.float64).transpose(0, 2, 1, 3).reshape(n, h * t, d), pl)
    o, lse = api.attn_merge(parts32, lses, out_dtype=torch.float32)
    o16, lse16 = api.attn_merge(parts32, lses)
    torch.cuda.synchronize()
    do, dl = compare(flat(o.cpu().numpy()), lse.cpu().numpy().reshape(h * t), om, lm, f"merge fp32->fp32 n={n}")
    assert do <= 1e-5 and dl <= 1e-5, (do, dl)
    assert torch.equal(o.to(torch.bfloat16).view(torch.int16), o16.view(torch.int16))
    assert torch.equal(lse, lse16)

    # bf16 partials, fp32 result
    o_bits = W.bf16_bits(o_p)
    parts16 = [dev_bf16(o_bits[i]) for i in range(n)]
    om, lm = oracle.merge(W.bf16_to_f32(o_bits).astype(np.float64).transpose(0, 2, 1, 3).reshape(n, h * t, d), pl)
    o, lse = api.attn_merge(parts16, lses, out_dtype=torch.float32)
    torch.cuda.synchronize()
    do, dl = compare(flat(o.cpu().numpy()), lse.cpu().numpy().reshape(h * t), om, lm, f"merge bf16->fp32 n={n}")
    assert do <= 1e-5 and dl <= 1e-5, (do, dl)


@pytest.mark.parametrize("q_chunk", [7])
def test_kv_split_fp32_partials_sampled(q_chunk):
    """The KV-split workload (8 key chunks of 8192, 32 heads, d 128) with fp32 partial
    outputs merged into bf16 and fp32 results, on sampled rows against the unsplit oracle."""
    import torch
    w = W.kv_split_q8192(q_chunk=q_chunk)
    c, nc = w.extra["chunk"], w.extra["n_chunks"]
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    plans = [api.Plan.from_slices(sl, c, c, w.hq, w.hkv, w.d).upload() for sl in w.extra["chunk_slices"]]
    say(f"kv split q8192 q_chunk={q_chunk}: 8 fp32-O partial forwards + merges")
    parts = [api.attn_fwd(q, k[t * c:(t + 1) * c], v[t * c:(t + 1) * c], plans[t], w.scale,
                          out_dtype=torch.float32) for t in range(nc)]
    o16, lse16 = api.attn_merge([p[0] for p in parts], [p[1] for p in parts])
    o32, lse32 = api.attn_merge([p[0] for p in parts], [p[1] for p in parts], out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = sample_rows(w, 192, 5)
    r = np.array(rows, np.int64)
    hs = torch.from_numpy(r[:, 0]).cuda()
    is_ = torch.from_numpy(r[:, 1]).cuda()
    o_ref, lse_ref = oracle.attn_fwd(w.q, w.k, w.v, w.slices, w.scale, rows=rows)
    compare(W.bf16_to_f32(host_bits(o16[is_, hs])), lse16[hs, is_].cpu().numpy(), o_ref, lse_ref,
            f"kv split q_chunk={q_chunk} fp32 partials -> bf16 O")
    compare(o32[is_, hs].cpu().numpy(), lse32[hs, is_].cpu().numpy(), o_ref, lse_ref,
            f"kv split q_chunk={q_chunk} fp32 partials -> fp32 O")
    for p in plans:
        p.close()
