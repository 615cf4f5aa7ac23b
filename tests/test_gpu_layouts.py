"""Strided layouts through the C ABI: Q, K and V as views of one packed QKV tensor, O and
LSE written into wider buffers, merge partials that are views.  The kernels address every
row through the token and head strides, so each result must equal, bit for bit, the same
call on contiguous copies (and the fp64 oracle within the stated tolerances)."""
import numpy as np
import pytest

import oracle
from block_sparse_flash_csr_amd import api
from block_sparse_flash_csr_amd import workloads as W

from gpu_helpers import compare, dev_bf16, host_bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    api.library()
    yield
    torch.cuda.synchronize()


def _packed(qb, kb, vb):
    """One [T, hq + 2 hkv, d] bf16 tensor holding Q | K | V per token, and its three views."""
    import torch
    sq, hq, d = qb.shape
    sk, hkv, _ = kb.shape
    assert sq == sk
    x = np.concatenate([qb, kb, vb], axis=1)
    t = dev_bf16(x)
    q, k, v = t[:, :hq], t[:, hq:hq + hkv], t[:, hq + hkv:]
    assert not q.is_contiguous() and q.stride(0) == (hq + 2 * hkv) * d
    return t, q, k, v


@pytest.mark.parametrize("hq,hkv,d", [(4, 4, 128), (8, 2, 128), (3, 1, 64)])
def test_forward_packed_qkv_and_strided_outputs(hq, hkv, d):
    import torch
    s = 777
    rng = np.random.default_rng(300 + hq + d)
    slices = W.random_slices(rng, s, s, 5) + [(0, s, 0, s, 1)]
    qb, kb, vb = W.random_inputs(rng, s, s, hq, hkv, d)
    say(f"packed QKV forward: s={s} hq={hq} hkv={hkv} d={d}")
    plan = api.Plan.from_slices(slices, s, s, hq, hkv, d).upload()
    o_ref, l_ref = api.attn_fwd(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), plan, 1.0 / np.sqrt(d))
    _, q, k, v = _packed(qb, kb, vb)
    o_big = torch.full((s, hq, d + 64), 7.0, dtype=torch.bfloat16, device="cuda")
    l_big = torch.full((hq, s + 40), 7.0, dtype=torch.float32, device="cuda")
    o, lse = api.attn_fwd(q, k, v, plan, 1.0 / np.sqrt(d), out=o_big[:, :, :d], lse=l_big[:, :s])
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse.nan_to_num(neginf=-1e30), l_ref.nan_to_num(neginf=-1e30))
    # nothing outside the views was written
    assert bool((o_big[:, :, d:].float() == 7.0).all()) and bool((l_big[:, s:] == 7.0).all())
    oo, lo = oracle.attn_fwd(qb, kb, vb, slices, 1.0 / np.sqrt(d))
    compare(W.bf16_to_f32(host_bits(o)), lse.cpu().numpy().T, oo, lo.T, "packed QKV forward")
    plan.close()


def test_backward_packed_inputs_equal_contiguous():
    import torch
    s, hq, hkv, d = 520, 4, 2, 128
    rng = np.random.default_rng(321)
    slices = W.random_slices(rng, s, s, 4) + [(0, s, 0, s, 1)]
    qb, kb, vb = W.random_inputs(rng, s, s, hq, hkv, d)
    gb = W.random_grad(rng, s, hq, d)
    say(f"packed QKV backward: s={s} hq={hq} hkv={hkv} d={d}")
    plan = api.Plan.from_slices(slices, s, s, hq, hkv, d).upload()
    qc, kc, vc = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    o, lse = api.attn_fwd(qc, kc, vc, plan, 1.0 / np.sqrt(d))
    g = dev_bf16(gb)
    ref = api.attn_bwd(qc, kc, vc, g, lse, plan, 1.0 / np.sqrt(d))
    _, q, k, v = _packed(qb, kb, vb)
    # dO as a view into a [T, 2 hq, d] buffer (beside O), LSE inside a wider one
    og = torch.cat([o, g], dim=1)
    l_big = torch.full((hq, s + 24), 3.0, dtype=torch.float32, device="cuda")
    l_big[:, :s] = lse
    got = api.attn_bwd(q, k, v, og[:, hq:], l_big[:, :s], plan, 1.0 / np.sqrt(d),
                       delta=torch.empty_like(l_big)[:, :s])
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(a, b), name
    plan.close()


def test_merge_of_strided_partials_equals_contiguous():
    import torch
    n, t, h, d = 5, 333, 6, 128
    rng = np.random.default_rng(55)
    parts = [W.bf16_bits(0.5 * rng.standard_normal((t, h, d), dtype=np.float32)) for _ in range(n)]
    lses = [rng.standard_normal((h, t)).astype(np.float32) * 3 for _ in range(n)]
    lses[2][1, 10:20] = -np.inf
    say(f"strided merge: n={n} t={t} h={h} d={d}")
    oc = [dev_bf16(p) for p in parts]
    lc = [torch.from_numpy(x).cuda() for x in lses]
    o_ref, l_ref = api.attn_merge(oc, lc)
    # partials as views of one [t, n*h, d] buffer (token stride n*h*d), LSE rows padded
    big = torch.cat(oc, dim=1)
    views = [big[:, i * h:(i + 1) * h] for i in range(n)]
    lbig = [torch.full((h, t + 8), 5.0, dtype=torch.float32, device="cuda") for _ in range(n)]
    for lb, x in zip(lbig, lc):
        lb[:, :t] = x
    o, lse = api.attn_merge(views, [lb[:, :t] for lb in lbig],
                            lse=torch.empty((h, t + 8), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse.nan_to_num(neginf=-1e30), l_ref.nan_to_num(neginf=-1e30))
    o_f = np.stack([W.bf16_to_f32(p).astype(np.float64) for p in parts])   # [n, t, h, d]
    po = o_f.transpose(0, 2, 1, 3).reshape(n, h * t, d)
    pl = np.stack(lses).reshape(n, h * t).astype(np.float64)
    om, lm = oracle.merge(po, pl)
    o_gpu = W.bf16_to_f32(host_bits(o)).transpose(1, 0, 2).reshape(h * t, d)
    compare(o_gpu, lse.contiguous().cpu().numpy().reshape(h * t), om, lm, "strided merge")


@pytest.mark.parametrize("d", [128, 64])
def test_fp32_outputs_as_views_equal_contiguous(d):
    """An fp32 O written into a wider fp32 buffer (its token stride padded by 4 elements,
    heads interleaved with a spare head), a backward from that view, and a merge of fp32
    partials that are views with an fp32 result view: each equal, bit for bit, to the same
    call on contiguous tensors."""
    import torch
    rng = np.random.default_rng(71 + d)
    s, hq, hkv = 300, 4, 2
    qb, kb, vb = W.random_inputs(rng, s, s, hq, hkv, d)
    gb = W.random_grad(rng, s, hq, d)
    q, k, v, g = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(gb)
    plan = api.Plan.from_slices(W.random_slices(rng, s, s, 6) + [(0, s, 0, s, 1)], s, s, hq, hkv, d).upload()
    say(f"fp32 outputs as views, d={d}")
    wide = torch.full((s, hq + 1, d + 4), float("nan"), dtype=torch.float32, device="cuda")
    ov = wide[:, 1:, :d]
    assert not ov.is_contiguous() and ov.stride(0) % 4 == 0 and ov.stride(1) % 4 == 0
    o_c, l_c = api.attn_fwd(q, k, v, plan, 0.1, out_dtype=torch.float32)
    o_v, l_v = api.attn_fwd(q, k, v, plan, 0.1, out=ov)
    g_c = api.attn_bwd(q, k, v, g, l_c, plan, 0.1, o=o_c)
    g_v = api.attn_bwd(q, k, v, g, l_v, plan, 0.1, o=ov)
    torch.cuda.synchronize()
    assert torch.equal(o_c, ov) and torch.equal(l_c, l_v)
    assert torch.isnan(wide[:, 0]).all() and torch.isnan(wide[:, :, d:]).all(), "wrote outside the view"
    for x, y in zip(g_c, g_v):
        assert torch.equal(x, y)
    # merge: three fp32 partials as views of one buffer, fp32 result as a view
    parts_buf = torch.from_numpy(rng.standard_normal((s, 3 * hq, d + 8)).astype(np.float32)).cuda()
    parts = [parts_buf[:, i * hq:(i + 1) * hq, :d] for i in range(3)]
    lses = [torch.from_numpy(rng.standard_normal((hq, s)).astype(np.float32)).cuda() for _ in range(3)]
    m_c, ml_c = api.attn_merge([p.contiguous() for p in parts], lses, out_dtype=torch.float32)
    res = torch.full((s, hq, d + 4), float("nan"), dtype=torch.float32, device="cuda")
    m_v, ml_v = api.attn_merge(parts, lses, out=res[:, :, :d])
    torch.cuda.synchronize()
    assert torch.equal(m_c, res[:, :, :d]) and torch.equal(ml_c, ml_v)
    assert torch.isnan(res[:, :, d:]).all(), "merge wrote outside the view"
    plan.close()
