"""The C-ABI library loads, exports every symbol include/bsfa.h declares, and rejects
bad arguments with the documented status codes (host-only calls, no GPU)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from block_sparse_flash_csr_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "bsfa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsfa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 14
    lib = api.library()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (bsfa_\w+)", out))
    assert set(names) <= exported


def test_status_strings():
    lib = api.library()
    for s in range(0, 9):
        assert lib.bsfa_status_str(s)


def _create(slices, sq, sk, hq=2, hkv=1, d=128, bq=128, bk=128):
    arr = (api.Slice * max(1, len(slices)))()
    for t, s in enumerate(slices):
        arr[t] = api.Slice(*s)
    h = ctypes.c_void_p()
    st = api.library().bsfa_plan_create(arr, len(slices), sq, sk, hq, hkv, d, bq, bk, ctypes.byref(h))
    if st == 0:
        api.library().bsfa_plan_destroy(h)
    return st


@pytest.mark.parametrize("slices,code", [
    ([(0, 10, 0, 10, 2)], 5),          # unknown type
    ([(5, 4, 0, 10, 0)], 5),           # q1 < q0
    ([(0, 10, 6, 5, 1)], 5),           # k1 < k0
    ([(0, 300, 0, 10, 0)], 5),         # q1 > sq
    ([(0, 10, 0, 300, 0)], 5),         # k1 > sk
    ([(-1, 10, 0, 10, 0)], 5),         # negative
])
def test_bad_slices_rejected(slices, code):
    assert _create(slices, 256, 256) == code


def test_bad_shapes_rejected():
    assert _create([], 256, 256, hq=3, hkv=2) == 2
    assert _create([], 256, 256, hq=0) == 1
    assert _create([], -1, 256) == 1
    assert _create([], 256, 256, bq=0) == 1
    lib = api.library()
    h = ctypes.c_void_p()
    assert lib.bsfa_plan_create(None, 1, 8, 8, 1, 1, 64, 128, 128, ctypes.byref(h)) == 1
    assert lib.bsfa_plan_create(None, 0, 8, 8, 1, 1, 64, 128, 128, None) == 1


def test_varlen_and_blocks_errors():
    lib = api.library()
    h = ctypes.c_void_p()
    cu = np.array([0, 10, 5], np.int32)   # decreasing
    assert lib.bsfa_plan_from_varlen(cu.ctypes.data_as(ctypes.c_void_p), 2, 1, 1, 1, 64, 128, 128,
                                     ctypes.byref(h)) == 5
    cu = np.array([3, 10], np.int32)      # does not start at 0
    assert lib.bsfa_plan_from_varlen(cu.ctypes.data_as(ctypes.c_void_p), 1, 1, 1, 1, 64, 128, 128,
                                     ctypes.byref(h)) == 5
    codes = np.array([[3]], np.uint8)     # unknown code
    assert lib.bsfa_plan_from_blocks(codes.ctypes.data_as(ctypes.c_void_p), 1, 1, 16, 16, 16, 16, 1,
                                     1, 64, 128, 128, ctypes.byref(h)) == 5


def test_forward_rejects_unuploaded_and_unsupported():
    """Checks that fail before any HIP call: no plan upload, unsupported tiles or head dim."""
    lib = api.library()
    p = api.Plan.from_slices([(0, 64, 0, 64, 1)], 64, 64, 1, 1, 128, bq=64, bk=64)
    t = api.Tensor(ctypes.c_void_p(16), 8, 8)
    lse = ctypes.c_void_p(16)
    st = lib.bsfa_attn_fwd(ctypes.byref(t), ctypes.byref(t), ctypes.byref(t), p.handle, 0.1,
                           ctypes.byref(t), lse, 64, None, 0, None)
    assert st == 4  # bq != 128
    p = api.Plan.from_slices([(0, 64, 0, 64, 1)], 64, 64, 1, 1, 96)
    st = lib.bsfa_attn_fwd(ctypes.byref(t), ctypes.byref(t), ctypes.byref(t), p.handle, 0.1,
                           ctypes.byref(t), lse, 64, None, 0, None)
    assert st == 4  # d = 96
    p = api.Plan.from_slices([(0, 64, 0, 64, 1)], 64, 64, 1, 1, 128)
    st = lib.bsfa_attn_fwd(ctypes.byref(t), ctypes.byref(t), ctypes.byref(t), p.handle, 0.1,
                           ctypes.byref(t), lse, 64, None, 0, None)
    assert st == 8  # not uploaded
    st = lib.bsfa_attn_fwd(ctypes.byref(t), ctypes.byref(t), ctypes.byref(t), p.handle, -1.0,
                           ctypes.byref(t), lse, 64, None, 0, None)
    assert st == 1  # non-positive scale


def test_forward_requires_a_workspace_for_split_rows():
    """A plan with split rows needs caller workspace of at least info.workspace_bytes (the
    plan itself holds none, so launches of one plan may overlap on several streams)."""
    lib = api.library()
    p = api.Plan.from_slices([(0, 128, 0, 65536, 1)], 128, 65536, 32, 8, 128)
    info = p.info()
    assert info["n_splits"] > 0 and info["workspace_bytes"] == info["n_units"] * 128 * 129 * 4
    t = api.Tensor(ctypes.c_void_p(16), 1024, 128)
    lse = ctypes.c_void_p(16)

    def call(ws, nbytes):
        return lib.bsfa_attn_fwd(ctypes.byref(t), ctypes.byref(t), ctypes.byref(t), p.handle, 0.1,
                                 ctypes.byref(t), lse, 128, ws, nbytes, None)

    assert call(None, 0) == 1                                        # no workspace
    assert call(ctypes.c_void_p(16), info["workspace_bytes"] - 16) == 1   # too small
    assert call(ctypes.c_void_p(24), info["workspace_bytes"]) == 3        # misaligned
    assert call(ctypes.c_void_p(16), -1) == 1
    assert call(ctypes.c_void_p(16), info["workspace_bytes"]) == 8        # then: not uploaded
    # a plan without split rows needs none
    q = api.Plan.from_slices([(0, 256, 0, 256, 1)], 256, 256, 2, 2, 128)
    assert q.info()["workspace_bytes"] == 0
    assert lib.bsfa_attn_fwd(ctypes.byref(t), ctypes.byref(t), ctypes.byref(t), q.handle, 0.1,
                             ctypes.byref(t), lse, 256, None, 0, None) == 8


def test_plans_past_the_addressing_limit_are_refused():
    """The kernels address entries (16 B) and pieces (32 B) with 32-bit byte offsets: a plan
    that reaches 2^27 non-empty tiles is refused rather than built and run wrong."""
    lib = api.library()
    h = ctypes.c_void_p()
    s = 16 * 16384            # causal at 16 x 16 tiles: 16384 * 16385 / 2 > 2^27 tiles
    one = (api.Slice * 1)(api.Slice(0, s, 0, s, 1))
    assert lib.bsfa_plan_create(one, 1, s, s, 1, 1, 128, 16, 16, ctypes.byref(h)) == 4
    assert not h.value
    s = 16 * 16383            # 16383 * 16384 / 2 = 134,209,536 < 2^27 tiles: accepted
    n_ok = 16383 * 16384 // 2
    assert n_ok < 1 << 27
    one = (api.Slice * 1)(api.Slice(0, s, 0, s, 1))
    assert lib.bsfa_plan_create(one, 1, s, s, 1, 1, 128, 16, 16, ctypes.byref(h)) == 0
    inf = api.PlanInfo()
    assert lib.bsfa_plan_get_info(h, ctypes.byref(inf)) == 0 and inf.nnz == n_ok
    lib.bsfa_plan_destroy(h)


def test_corrupted_plans_are_refused_before_upload():
    """tests/c_abi/plan_check (built by build()) corrupts one plan field at a time through
    the library's internal layout; the upload's host-side check must refuse each plan
    with BSFA_ERR_PLAN before any device work, and pass the intact plans."""
    import subprocess
    exe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "plan_check")
    if not os.path.exists(exe):
        pytest.fail(f"{exe} is missing: run build() first")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert sum(line.startswith("ok") for line in r.stdout.splitlines()) == 18


def test_merge_binding_rejects_strided_head_dim_and_short_lse():
    """The merge kernel reads partials with a contiguous head dim and LSE rows covering
    every merged token; the binding refuses other views before any device call."""
    import torch
    base = torch.zeros((8, 2, 256), dtype=torch.bfloat16)
    parts = [base[..., ::2], base[..., ::2]]          # head dim stride 2
    lses = [torch.zeros((2, 8)), torch.zeros((2, 8))]
    with pytest.raises(ValueError):
        api.attn_merge(parts, lses)
    parts = [torch.zeros((8, 2, 128), dtype=torch.bfloat16)] * 2
    short = [torch.zeros((2, 16))[:, :4]] * 2         # 4 tokens of LSE for 8 merged tokens
    with pytest.raises(ValueError):
        api.attn_merge(parts, short)


def test_bindings_refuse_host_tensors_and_short_outputs():
    """Every tensor a kernel touches must be a CUDA tensor of the current device, and the
    outputs must cover the call's rows; the bindings refuse the rest before any device
    call (here all tensors are host tensors, so the shape checks must come first)."""
    import torch
    sq, sk, hq, hkv, d = 100, 90, 2, 1, 64
    plan = api.Plan.from_slices([(0, sq, 0, sk, 1)], sq, sk, hq, hkv, d)
    q = torch.zeros((sq, hq, d), dtype=torch.bfloat16)
    k = v = torch.zeros((sk, hkv, d), dtype=torch.bfloat16)
    lse = torch.zeros((hq, sq))
    with pytest.raises(ValueError, match="lse covers"):
        api.attn_fwd(q, k, v, plan, 0.1, lse=torch.zeros((hq, 256))[:, :sq - 1])
    with pytest.raises(ValueError, match="CUDA tensor"):
        api.attn_fwd(q, k, v, plan, 0.1)
    with pytest.raises(ValueError, match="lse covers"):
        api.attn_bwd(q, k, v, q, lse[:, :sq - 1], plan, 0.1)
    with pytest.raises(ValueError, match="CUDA tensor"):
        api.attn_bwd(q, k, v, q, lse, plan, 0.1)
    plan.close()
    parts = [torch.zeros((8, 2, 128), dtype=torch.bfloat16)] * 2
    lses = [torch.zeros((2, 8))] * 2
    with pytest.raises(ValueError, match="out shape"):
        api.attn_merge(parts, lses, out=torch.zeros((7, 2, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="lse must be"):
        api.attn_merge(parts, lses, lse=torch.zeros((2, 16))[:, :7])
    with pytest.raises(ValueError, match="CUDA tensor"):
        api.attn_merge(parts, lses)


def test_rescale_threshold_setting():
    """The conditional-rescale threshold accepts 0..64 (log2 units) and refuses the rest."""
    lib = api.library()
    assert api.rescale_threshold() == 8.0
    try:
        for bad in (-0.5, 64.5, float("nan"), float("inf")):
            assert lib.bsfa_set_rescale_threshold(bad) == 1
        assert api.rescale_threshold() == 8.0
        api.set_rescale_threshold(0.0)
        assert api.rescale_threshold() == 0.0
        api.set_rescale_threshold(64.0)
        assert api.rescale_threshold() == 64.0
    finally:
        api.set_rescale_threshold(8.0)


def test_merge_rejects_bad_arguments():
    lib = api.library()
    t = api.Tensor(ctypes.c_void_p(16), 1024, 128)
    ptrs = (ctypes.c_void_p * 2)(16, 32)
    lptr = (ctypes.c_void_p * 2)(16, 32)
    assert lib.bsfa_attn_merge(ptrs, lptr, 0, 1024, 128, 64, 64, 8, 128, ctypes.byref(t),
                               ctypes.c_void_p(16), None) == 1
    assert lib.bsfa_attn_merge(ptrs, lptr, 17, 1024, 128, 64, 64, 8, 128, ctypes.byref(t),
                               ctypes.c_void_p(16), None) == 1
    assert lib.bsfa_attn_merge(ptrs, lptr, 2, 1024, 128, 64, 64, 8, 96, ctypes.byref(t),
                               ctypes.c_void_p(16), None) == 4
    assert lib.bsfa_attn_merge(ptrs, lptr, 2, 1020, 128, 64, 64, 8, 128, ctypes.byref(t),
                               ctypes.c_void_p(16), None) == 3
    bad = (ctypes.c_void_p * 2)(16, 40)
    assert lib.bsfa_attn_merge(bad, lptr, 2, 1024, 128, 64, 64, 8, 128, ctypes.byref(t),
                               ctypes.c_void_p(16), None) == 3
    assert lib.bsfa_attn_merge(ptrs, lptr, 2, 1024, 128, 10, 64, 8, 128, ctypes.byref(t),
                               ctypes.c_void_p(16), None) == 1
    # nothing to merge: no pointer is read, the call succeeds (still checking d)
    empty = api.Tensor(ctypes.c_void_p(None), 1024, 128)
    nulls = (ctypes.c_void_p * 2)(None, None)
    assert lib.bsfa_attn_merge(nulls, nulls, 2, 1024, 128, 0, 0, 8, 128, ctypes.byref(empty), None, None) == 0
    assert lib.bsfa_attn_merge(nulls, nulls, 2, 1024, 128, 0, 0, 8, 96, ctypes.byref(empty), None, None) == 4


def test_typed_entry_points_reject_bad_types_and_strides():
    """The fp32-output forms: unknown element types, and fp32 strides that are not
    16-byte multiples, fail before any HIP call; an fp32 stride of 4 elements passes the
    stride check (the call then stops at the missing result pointer)."""
    lib = api.library()
    t = api.Tensor(ctypes.c_void_p(16), 1024, 128)
    ptrs = (ctypes.c_void_p * 2)(16, 32)
    lptr = (ctypes.c_void_p * 2)(16, 32)
    buf = ctypes.c_void_p(16)

    def merge(pdt, odt, p_st=1024, o=t):
        return lib.bsfa_attn_merge_typed(ptrs, pdt, lptr, 2, p_st, 128, 64, 64, 8, 128, ctypes.byref(o), odt,
                                         buf, None)

    assert merge(2, 0) == 1 and merge(0, -1) == 1            # unknown types
    assert merge(1, 0, p_st=1022) == 3                         # fp32 partial rows not 16-byte aligned
    assert merge(0, 0, p_st=1020) == 3                         # bf16 stride: multiple of 8 needed
    assert merge(1, 1, o=api.Tensor(ctypes.c_void_p(16), 1026, 128)) == 3
    nul = api.Tensor(ctypes.c_void_p(None), 1020, 128)
    assert merge(1, 1, p_st=1020, o=nul) == 1                  # strides accepted, no result pointer
    p = api.Plan.from_slices([(0, 64, 0, 64, 1)], 64, 64, 1, 1, 128)
    tp = [ctypes.byref(api.Tensor(ctypes.c_void_p(16), 128, 128))] * 3
    o = api.Tensor(ctypes.c_void_p(16), 128, 128)
    for bad in (2, -1, 7):
        assert lib.bsfa_attn_fwd_typed(*tp, p.handle, 0.1, ctypes.byref(o), bad, buf, 64, None, 0, None) == 1
    assert lib.bsfa_attn_fwd_typed(*tp, p.handle, 0.1, ctypes.byref(o), 1, buf, 64, None, 0, None) == 8  # not uploaded


def test_backward_rejects_bad_arguments():
    """Checks of the gradient entry that fail before any HIP call."""
    lib = api.library()
    t = api.Tensor(ctypes.c_void_p(16), 8, 8)
    buf = ctypes.c_void_p(16)
    tp = [ctypes.byref(t)] * 4

    def call(plan, scale=0.1, lse=buf, dq=buf, delta=buf):
        return lib.bsfa_attn_bwd(*tp, lse, 64, plan.handle, scale, dq, buf, buf, delta, None)

    p = api.Plan.from_slices([(0, 64, 0, 64, 1)], 64, 64, 1, 1, 128, bq=64, bk=64)
    assert call(p) == 4                # tiles other than 128 x 128
    p = api.Plan.from_slices([(0, 64, 0, 64, 1)], 64, 64, 1, 1, 96)
    assert call(p) == 4                # d = 96
    p = api.Plan.from_slices([(0, 64, 0, 64, 1)], 64, 64, 1, 1, 128)
    assert call(p, scale=0.0) == 1     # non-positive scale
    assert call(p, lse=None) == 1      # no LSE
    assert call(p, delta=None) == 1    # no delta scratch
    assert call(p) == 8                # not uploaded
    assert lib.bsfa_attn_bwd_o32(*tp, None, buf, 64, p.handle, 0.1, buf, buf, buf, buf, None) == 1  # no O
    o = api.Tensor(ctypes.c_void_p(16), 8, 8)
    assert lib.bsfa_attn_bwd_o32(*tp, ctypes.byref(o), buf, 64, p.handle, 0.1, buf, buf, buf, buf, None) == 8


def test_device_compiler_rejects_bad_arguments():
    """Checks of bsfa_dcsr_build that fail before any HIP call."""
    lib = api.library()
    h = ctypes.c_void_p()
    one = (api.Slice * 1)(api.Slice(0, 10, 0, 10, 0))
    assert lib.bsfa_dcsr_build(one, 1, 10, 10, 128, 512, None, ctypes.byref(h)) == 4   # bk > 256
    bad = (api.Slice * 1)(api.Slice(0, 10, 0, 20, 0))
    assert lib.bsfa_dcsr_build(bad, 1, 10, 10, 128, 128, None, ctypes.byref(h)) == 5   # k1 > sk
    bad = (api.Slice * 1)(api.Slice(0, 10, 0, 10, 3))
    assert lib.bsfa_dcsr_build(bad, 1, 10, 10, 128, 128, None, ctypes.byref(h)) == 5   # unknown type
    assert lib.bsfa_dcsr_build(one, 1, 10, 10, 0, 128, None, ctypes.byref(h)) == 1     # bq = 0
    assert lib.bsfa_dcsr_build(one, 1, 10, 10, 128, 128, None, None) == 1              # no out
    assert lib.bsfa_dcsr_build(None, 1, 10, 10, 128, 128, None, ctypes.byref(h)) == 1  # no slices
    assert lib.bsfa_plan_from_dcsr(None, 2, 1, 128, ctypes.byref(h)) == 1              # no csr
    assert lib.bsfa_plan_from_dcsr(None, 2, 1, 128, None) == 1                         # no out


def test_block_code_device_compiler_rejects_bad_arguments():
    """Checks of bsfa_dcsr_build_blocks that fail before any HIP call."""
    lib = api.library()
    h = ctypes.c_void_p()
    codes = np.zeros((3, 3), np.uint8)
    codes[2, 2] = 3
    assert lib.bsfa_dcsr_build_blocks(api._ptr(codes), 3, 3, 384, 384, 128, 128, None, ctypes.byref(h)) == 5
    codes[2, 2] = 1
    assert lib.bsfa_dcsr_build_blocks(api._ptr(codes), 3, 3, 384, 384, 0, 128, None, ctypes.byref(h)) == 1
    assert lib.bsfa_dcsr_build_blocks(api._ptr(codes), 3, 3, -1, 384, 128, 128, None, ctypes.byref(h)) == 1
    assert lib.bsfa_dcsr_build_blocks(None, 3, 3, 384, 384, 128, 128, None, ctypes.byref(h)) == 1
    assert lib.bsfa_dcsr_build_blocks(api._ptr(codes), 3, 3, 384, 384, 128, 128, None, None) == 1
    # a code above 2 outside the tile grid is refused too (as bsfa_plan_from_blocks does)
    big = np.zeros((5, 5), np.uint8)
    big[4, 4] = 7
    assert lib.bsfa_dcsr_build_blocks(api._ptr(big), 5, 5, 100, 100, 128, 128, None, ctypes.byref(h)) == 5
    assert not h.value
