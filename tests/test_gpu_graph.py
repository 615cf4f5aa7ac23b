"""The forwards replayed from a captured HIP graph (torch.cuda.graph): the no-allocation
forward (its use case: callers under graph capture) and the caller-workspace forward of
a plan with split rows, each replayed several times with new inputs copied in eagerly
between replays, every replay bit-identical to an eager call on the same inputs."""
import ctypes

import numpy as np
import pytest

from block_sparse_flash_csr_amd import api
from block_sparse_flash_csr_amd import workloads as W

from gpu_helpers import dev_bf16, say

pytestmark = pytest.mark.gpu


def _tensor(t):
    return api.Tensor(ctypes.c_void_p(t.data_ptr()), t.stride(0), t.stride(1))


def _noalloc_into(q, k, v, plan, scale, o, lse):
    tq, tk, tv, to = _tensor(q), _tensor(k), _tensor(v), _tensor(o)
    st = api.library().bsfa_attn_fwd_noalloc(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), plan.handle,
                                              float(scale), ctypes.byref(to), ctypes.c_void_p(lse.data_ptr()),
                                              lse.stride(0), api._stream_handle())
    assert st == 0, api.BsfaError("bsfa_attn_fwd_noalloc", st)


@pytest.mark.parametrize("noalloc", [True, False])
def test_forward_replayed_from_a_graph(noalloc):
    import torch
    rng = np.random.default_rng(91 if noalloc else 92)
    sq, sk, hq, hkv, d = 256, 20000, 8, 2, 128
    slices = [(0, sq, 0, sk, 1), (0, 40, 3000, 3100, 0)]
    plan = api.Plan.from_slices(slices, sq, sk, hq, hkv, d).upload()
    info = plan.info()
    assert info["n_splits"] > 0, info
    say(f"graph replay ({'no-alloc' if noalloc else 'caller workspace'}): sq={sq} sk={sk} hq={hq} hkv={hkv} "
        f"d={d}, {info['n_splits']} split rows")
    scale = 1.0 / np.sqrt(d)
    qb, kb, vb = W.random_inputs(rng, sq, sk, hq, hkv, d)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    o_g = torch.empty((sq, hq, d), dtype=torch.bfloat16, device="cuda")
    l_g = torch.empty((hq, sq), dtype=torch.float32, device="cuda")
    ws = None if noalloc else api.workspace_for(plan)

    def fwd(o, lse):
        if noalloc:
            _noalloc_into(q, k, v, plan, scale, o, lse)
        else:
            api.attn_fwd(q, k, v, plan, scale, out=o, lse=lse, workspace=ws)

    # eager warm-up: the plan is resident and the static workspace's address known
    fwd(o_g, l_g)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(o_g, l_g)
    torch.cuda.synchronize()
    o_e = torch.empty_like(o_g)
    l_e = torch.empty_like(l_g)
    for r in range(3):
        # new inputs, copied in by the program's own eager work
        qn, kn, vn = W.random_inputs(np.random.default_rng(1000 * r + 7), sq, sk, hq, hkv, d)
        q.copy_(dev_bf16(qn))
        k.copy_(dev_bf16(kn))
        v.copy_(dev_bf16(vn))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        fwd(o_e, l_e)
        torch.cuda.synchronize()
        assert torch.equal(o_g.view(torch.int16), o_e.view(torch.int16)), f"replay {r}: O differs from eager"
        assert torch.equal(l_g, l_e), f"replay {r}: LSE differs from eager"
        say(f"replay {r}: bit-identical to the eager call")
    del g
    plan.close()


@pytest.mark.parametrize("fp32", [False, True])
def test_backward_and_merge_replayed_from_a_graph(fp32):
    """The backward kernels and the merge kernel captured once and replayed with new
    inputs; each replay bit-identical to eager calls (none of them clears memory with a
    memset node: every output element is written by a kernel).  fp32: the backward from
    the forward's fp32 O (two kernels) and the merge of fp32 partials into an fp32 result."""
    import torch
    rng = np.random.default_rng(93)
    sq, sk, hq, hkv, d = 700, 700, 4, 2, 128
    slices = [(0, sq, 0, sk, 1)]
    plan = api.Plan.from_slices(slices, sq, sk, hq, hkv, d).upload()
    scale = 1.0 / np.sqrt(d)
    say(f"graph replay (backward + merge): sq={sq} sk={sk} hq={hq} hkv={hkv} d={d}")
    qb, kb, vb = W.random_inputs(rng, sq, sk, hq, hkv, d)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    g_o = dev_bf16(W.random_grad(rng, sq, hq, d))
    o, lse = api.attn_fwd(q, k, v, plan, scale, out_dtype=torch.float32 if fp32 else None)
    o_in = o if fp32 else None
    parts_o = [torch.empty_like(o) for _ in range(3)]
    parts_l = [torch.empty_like(lse) for _ in range(3)]
    bufs = {n: torch.empty(s, dtype=torch.float32, device="cuda")
            for n, s in (("dq", (sq, hq, d)), ("dk", (sk, hkv, d)), ("dv", (sk, hkv, d)), ("delta", (hq, sq)))}
    m_o, m_l = torch.empty_like(o), torch.empty_like(lse)

    def work(dst, mo, ml):
        api.attn_bwd(q, k, v, g_o, lse, plan, scale, dq=dst["dq"], dk=dst["dk"], dv=dst["dv"], delta=dst["delta"],
                     o=o_in)
        api.attn_merge(parts_o, parts_l, out=mo, lse=ml)

    work(bufs, m_o, m_l)   # eager warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work(bufs, m_o, m_l)
    torch.cuda.synchronize()
    ref = {n: torch.empty_like(t) for n, t in bufs.items()}
    r_o, r_l = torch.empty_like(o), torch.empty_like(lse)
    for r in range(3):
        rr = np.random.default_rng(2000 + r)
        qn, kn, vn = W.random_inputs(rr, sq, sk, hq, hkv, d)
        q.copy_(dev_bf16(qn))
        k.copy_(dev_bf16(kn))
        v.copy_(dev_bf16(vn))
        g_o.copy_(dev_bf16(W.random_grad(rr, sq, hq, d)))
        api.attn_fwd(q, k, v, plan, scale, out=o, lse=lse)
        for t in range(3):
            parts_o[t].copy_(dev_bf16(W.random_grad(rr, sq, hq, d)))     # (converted when fp32)
            parts_l[t].copy_(torch.from_numpy(rr.standard_normal((hq, sq)).astype(np.float32)).cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        work(ref, r_o, r_l)
        torch.cuda.synchronize()
        for n in bufs:
            assert torch.equal(bufs[n], ref[n]), f"replay {r}: {n} differs from eager"
        bits = torch.int32 if fp32 else torch.int16
        assert torch.equal(m_o.view(bits), r_o.view(bits)) and torch.equal(m_l, r_l), \
            f"replay {r}: merge differs from eager"
        say(f"replay {r}: gradients and merge bit-identical to the eager calls")
    del g
    plan.close()
