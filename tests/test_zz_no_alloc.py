"""bsfa_attn_fwd_noalloc, the forward for callers that cannot allocate: the split rows'
partial results go to the library's static per-GPU workspace instead of a caller buffer.
Called through the C ABI and checked bit for bit against bsfa_attn_fwd with a caller
workspace (the same kernels), and against the fp64 oracle at the stated tolerances, on
two calls in a row: the second with a smaller problem, whose parts must overwrite
everything they read of the workspace the first call left behind."""
import ctypes

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


def _tensor(t):
    return api.Tensor(ctypes.c_void_p(t.data_ptr()), t.stride(0), t.stride(1))


def fwd_noalloc(q, k, v, plan, scale):
    import torch
    sq, hq, d = q.shape
    o = torch.empty((sq, hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((hq, sq), dtype=torch.float32, device="cuda")
    tq, tk, tv, to = _tensor(q), _tensor(k), _tensor(v), _tensor(o)
    st = api.library().bsfa_attn_fwd_noalloc(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), plan.handle,
                                              float(scale), ctypes.byref(to), ctypes.c_void_p(lse.data_ptr()),
                                              lse.stride(0), api._stream_handle())
    assert st == 0, api.BsfaError("bsfa_attn_fwd_noalloc", st)
    return o, lse


# (seed, sq, sk, hq, hkv, d, extra slices): the second problem is smaller than the first
CASES = [
    (81, 256, 20000, 8, 2, 128, [(0, 40, 3000, 3100, 0)]),
    (82, 100, 7000, 4, 1, 64, [(50, 100, 0, 500, 0)]),
]


def test_noalloc_equals_caller_workspace_on_two_calls():
    import torch
    prev_ws = None
    for seed, sq, sk, hq, hkv, d, extra in CASES:
        rng = np.random.default_rng(seed)
        slices = [(0, sq, 0, sk, 1)] + extra
        qb, kb, vb = W.random_inputs(rng, sq, sk, hq, hkv, d)
        q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
        plan = api.Plan.from_slices(slices, sq, sk, hq, hkv, d).upload()
        info = plan.info()
        assert info["n_splits"] > 0 and 0 < info["workspace_bytes"] <= api.STATIC_WORKSPACE_BYTES, info
        if prev_ws is not None:
            assert info["workspace_bytes"] < prev_ws
        prev_ws = info["workspace_bytes"]
        say(f"no-alloc forward: sq={sq} sk={sk} hq={hq} hkv={hkv} d={d}: {info['n_splits']} split rows, "
            f"{info['n_units']} units, workspace {info['workspace_bytes']} B")
        scale = 1.0 / np.sqrt(d)
        o_ref, l_ref = api.attn_fwd(q, k, v, plan, scale)
        o, lse = fwd_noalloc(q, k, v, plan, scale)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), "O differs from the caller-workspace call"
        assert torch.equal(lse, l_ref), "LSE differs from the caller-workspace call"
        oo, lo = oracle.attn_fwd(qb, kb, vb, slices, scale)
        compare(W.bf16_to_f32(host_bits(o)), lse.cpu().numpy().T, oo, lo.T, f"no-alloc forward sq={sq} sk={sk}")
        plan.close()


def test_noalloc_without_split_rows():
    """A plan without split rows never touches the static workspace."""
    import torch
    rng = np.random.default_rng(83)
    sq = sk = 700
    slices = [(0, sq, 0, sk, 1)]
    qb, kb, vb = W.random_inputs(rng, sq, sk, 4, 2, 128)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    plan = api.Plan.from_slices(slices, sq, sk, 4, 2, 128).upload()
    assert plan.info()["workspace_bytes"] == 0
    o_ref, l_ref = api.attn_fwd(q, k, v, plan, 0.09)
    o, lse = fwd_noalloc(q, k, v, plan, 0.09)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(lse, l_ref)
    plan.close()


def test_noalloc_refuses_plans_beyond_the_static_workspace():
    """About 500 split-row parts at d = 128 fill the 32 MiB workspace; a plan that needs
    more is refused with BSFA_ERR_UNSUPPORTED before any device work."""
    import torch
    plan = api.Plan.from_slices([(0, 128, 0, 262144, 1)], 128, 262144, 64, 8, 128).upload()
    info = plan.info()
    assert info["workspace_bytes"] > api.STATIC_WORKSPACE_BYTES, info
    q = torch.zeros((128, 64, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((262144, 8, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((64, 128), dtype=torch.float32, device="cuda")
    tq, tk, to = _tensor(q), _tensor(kv), _tensor(o)
    st = api.library().bsfa_attn_fwd_noalloc(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tk), plan.handle, 0.1,
                                              ctypes.byref(to), ctypes.c_void_p(lse.data_ptr()), 128,
                                              api._stream_handle())
    assert st == 4
    plan.close()
