"""Thin Python binding over libbsfa.so (include/bsfa.h): argument marshalling only.

Every step of the path (mask compile, schedule, forward, merge) runs inside the
library.  torch supplies device memory and the current stream.  When the library
is missing this module raises: there is no Python or CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsfa.so")

BSFA_FULL, BSFA_CAUSAL = 0, 1
TILE_FULL, TILE_PARTIAL = 1, 2
MERGE_MAX_PARTS = 16
STATIC_WORKSPACE_BYTES = 32 << 20     # bsfa_attn_fwd_noalloc's per-GPU workspace

_STATUS = {0: "ok", 1: "invalid argument", 2: "shape mismatch", 3: "misaligned pointer or stride",
           4: "unsupported head dim or tile size", 5: "invalid mask", 6: "out of memory",
           7: "HIP runtime error", 8: "plan not uploaded to the current device",
           9: "plan metadata failed its consistency check"}


class BsfaError(RuntimeError):
    def __init__(self, call, status):
        super().__init__(f"{call}: {_STATUS.get(status, status)} (status {status})")
        self.status = status


class Slice(ctypes.Structure):
    _fields_ = [("q0", ctypes.c_int32), ("q1", ctypes.c_int32), ("k0", ctypes.c_int32),
                ("k1", ctypes.c_int32), ("type", ctypes.c_int32)]


class Tensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride_tok", ctypes.c_int64),
                ("stride_head", ctypes.c_int64)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("sq", ctypes.c_int32), ("sk", ctypes.c_int32), ("hq", ctypes.c_int32),
                ("hkv", ctypes.c_int32), ("d", ctypes.c_int32), ("bq", ctypes.c_int32),
                ("bk", ctypes.c_int32), ("n_qtiles", ctypes.c_int32), ("n_ktiles", ctypes.c_int32),
                ("nnz", ctypes.c_int64), ("n_full", ctypes.c_int64), ("n_partial", ctypes.c_int64),
                ("n_pieces", ctypes.c_int64), ("pairs", ctypes.c_int64), ("n_items", ctypes.c_int32),
                ("n_bins", ctypes.c_int32), ("makespan", ctypes.c_double),
                ("total_cost", ctypes.c_double), ("uploaded", ctypes.c_int32),
                ("n_units", ctypes.c_int32), ("n_splits", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64)]


_lib = None


def library():
    """Load libbsfa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m block_sparse_flash_csr_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    PP = ctypes.POINTER(ctypes.c_void_p)
    lib.bsfa_plan_create.argtypes = [P, I32, I32, I32, I32, I32, I32, I32, I32, PP]
    lib.bsfa_plan_from_varlen.argtypes = [P, I32, I32, I32, I32, I32, I32, I32, PP]
    lib.bsfa_plan_from_blocks.argtypes = [P, I32, I32, I32, I32, I32, I32, I32, I32, I32, I32, I32, PP]
    lib.bsfa_plan_upload.argtypes = [P, P]
    lib.bsfa_plan_destroy.argtypes = [P]
    lib.bsfa_plan_destroy.restype = None
    lib.bsfa_plan_get_info.argtypes = [P, ctypes.POINTER(PlanInfo)]
    lib.bsfa_plan_export_csr.argtypes = [P, P, P, P, I64, ctypes.POINTER(I64)]
    lib.bsfa_plan_export_schedule.argtypes = [P, P, P, P]
    lib.bsfa_plan_export_units.argtypes = [P, P]
    lib.bsfa_tile_cost.argtypes = [I32, ctypes.c_double]
    lib.bsfa_tile_cost.restype = ctypes.c_double
    lib.bsfa_imbalance_bound.argtypes = [ctypes.c_double, I32]
    lib.bsfa_imbalance_bound.restype = ctypes.c_double
    lib.bsfa_lpt_assign.argtypes = [P, I32, I32, P, P]
    lib.bsfa_lpt_assign.restype = ctypes.c_double
    lib.bsfa_attn_fwd.argtypes = [ctypes.POINTER(Tensor)] * 3 + [P, ctypes.c_float,
                                                                 ctypes.POINTER(Tensor), P, I64, P, I64, P]
    lib.bsfa_attn_fwd_noalloc.argtypes = [ctypes.POINTER(Tensor)] * 3 + [P, ctypes.c_float,
                                                                         ctypes.POINTER(Tensor), P, I64, P]
    lib.bsfa_attn_merge.argtypes = [P, P, I32, I64, I64, I64, I32, I32, I32,
                                    ctypes.POINTER(Tensor), P, P]
    lib.bsfa_attn_fwd_typed.argtypes = [ctypes.POINTER(Tensor)] * 3 + [P, ctypes.c_float,
                                                                       ctypes.POINTER(Tensor), I32, P, I64, P,
                                                                       I64, P]
    lib.bsfa_attn_merge_typed.argtypes = [P, I32, P, I32, I64, I64, I64, I32, I32, I32,
                                          ctypes.POINTER(Tensor), I32, P, P]
    lib.bsfa_attn_bwd.argtypes = [ctypes.POINTER(Tensor)] * 4 + [P, I64, P, ctypes.c_float,
                                                                 P, P, P, P, P]
    lib.bsfa_attn_bwd_o32.argtypes = [ctypes.POINTER(Tensor)] * 5 + [P, I64, P, ctypes.c_float,
                                                                     P, P, P, P, P]
    lib.bsfa_plan_export_pieces.argtypes = [P, P, P, I64]
    lib.bsfa_dcsr_build.argtypes = [P, I32, I32, I32, I32, I32, P, PP]
    lib.bsfa_dcsr_build_blocks.argtypes = [P, I32, I32, I32, I32, I32, I32, P, PP]
    lib.bsfa_dcsr_view_get.argtypes = [P, ctypes.POINTER(DcsrView)]
    lib.bsfa_dcsr_export.argtypes = [P, P, P, P, P, P, I64, I64]
    lib.bsfa_dcsr_destroy.argtypes = [P]
    lib.bsfa_plan_from_dcsr.argtypes = [P, I32, I32, I32, PP]
    lib.bsfa_dcsr_destroy.restype = None
    lib.bsfa_set_rescale_threshold.argtypes = [ctypes.c_float]
    lib.bsfa_set_rescale_threshold.restype = I32
    lib.bsfa_get_rescale_threshold.argtypes = []
    lib.bsfa_get_rescale_threshold.restype = ctypes.c_float
    lib.bsfa_status_str.argtypes = [I32]
    lib.bsfa_status_str.restype = ctypes.c_char_p
    for name in ("bsfa_plan_create", "bsfa_plan_from_varlen", "bsfa_plan_from_blocks",
                 "bsfa_plan_upload", "bsfa_plan_get_info", "bsfa_plan_export_csr",
                 "bsfa_plan_export_schedule", "bsfa_plan_export_units", "bsfa_attn_fwd",
                 "bsfa_attn_fwd_noalloc", "bsfa_attn_fwd_typed", "bsfa_attn_merge_typed", "bsfa_attn_bwd_o32",
                 "bsfa_attn_merge", "bsfa_attn_bwd", "bsfa_plan_export_pieces", "bsfa_dcsr_build",
                 "bsfa_dcsr_build_blocks", "bsfa_dcsr_view_get", "bsfa_dcsr_export", "bsfa_plan_from_dcsr"):
        getattr(lib, name).restype = I32
    _lib = lib
    return lib


def _check(call, status):
    if status != 0:
        raise BsfaError(call, status)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def slice_array(slices) -> np.ndarray:
    """Slices (q0, q1, k0, k1, type) as a contiguous int32 [n, 5] array (bsfa_slice layout).
    An array already in that layout is passed through without a copy."""
    if (isinstance(slices, np.ndarray) and slices.dtype == np.int32 and slices.ndim == 2
            and slices.shape[1] == 5 and slices.flags.c_contiguous):
        return slices
    arr = np.ascontiguousarray(np.asarray(slices, dtype=np.int64).reshape(-1, 5))
    if arr.size and (arr.min() < np.iinfo(np.int32).min or arr.max() > np.iinfo(np.int32).max):
        raise ValueError("slice bounds must fit in int32")
    return np.ascontiguousarray(arr.astype(np.int32))


def _stream_handle(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


class DcsrView(ctypes.Structure):
    _fields_ = [("row_ptr", ctypes.c_void_p), ("col", ctypes.c_void_p), ("tag", ctypes.c_void_p),
                ("piece_ptr", ctypes.c_void_p), ("pieces", ctypes.c_void_p),
                ("n_qtiles", ctypes.c_int32), ("n_ktiles", ctypes.c_int32),
                ("nnz", ctypes.c_int64), ("n_full", ctypes.c_int64), ("n_partial", ctypes.c_int64),
                ("n_pieces", ctypes.c_int64), ("pairs", ctypes.c_int64), ("touches", ctypes.c_int64)]


class DeviceCsr:
    """Tile CSR compiled on the GPU (bsfa_dcsr_build); `view()` waits for it."""

    def __init__(self, slices, sq, sk, bq=128, bk=128, stream=None):
        arr = slice_array(slices)
        h = ctypes.c_void_p()
        _check("bsfa_dcsr_build", library().bsfa_dcsr_build(_ptr(arr), len(arr), sq, sk, bq, bk,
                                                             _stream_handle(stream), ctypes.byref(h)))
        self._h = h

    @classmethod
    def from_blocks(cls, codes, sq, sk, bq=128, bk=128, stream=None) -> "DeviceCsr":
        """Tile CSR of a block-code map over (bq x bk) blocks (0 empty, 1 full, 2 causal),
        compiled on the GPU (bsfa_dcsr_build_blocks): the CSR Plan.from_blocks builds
        with blocks equal to tiles."""
        c = np.ascontiguousarray(codes, dtype=np.uint8)
        assert c.ndim == 2
        h = ctypes.c_void_p()
        _check("bsfa_dcsr_build_blocks", library().bsfa_dcsr_build_blocks(
            _ptr(c), c.shape[0], c.shape[1], sq, sk, bq, bk, _stream_handle(stream), ctypes.byref(h)))
        obj = cls.__new__(cls)
        obj._h = h
        return obj

    def view(self) -> dict:
        v = DcsrView()
        _check("bsfa_dcsr_view_get", library().bsfa_dcsr_view_get(self._h, ctypes.byref(v)))
        return {f: getattr(v, f) for f, _ in DcsrView._fields_}

    def export(self):
        """(row_ptr, col, tag, piece_ptr, pieces [n, 5]) as numpy arrays."""
        v = self.view()
        row_ptr = np.zeros(v["n_qtiles"] + 1, np.int32)
        col = np.zeros(max(1, v["nnz"]), np.int32)
        tag = np.zeros(max(1, v["nnz"]), np.uint8)
        piece_ptr = np.zeros(v["nnz"] + 1, np.int32)
        pieces = np.zeros((max(1, v["n_pieces"]), 5), np.int32)
        _check("bsfa_dcsr_export", library().bsfa_dcsr_export(
            self._h, _ptr(row_ptr), _ptr(col), _ptr(tag), _ptr(piece_ptr), _ptr(pieces),
            v["nnz"], v["n_pieces"]))
        return row_ptr, col[:v["nnz"]], tag[:v["nnz"]], piece_ptr, pieces[:v["n_pieces"]]

    def plan(self, hq, hkv, d) -> "Plan":
        """The plan over this CSR, built on the device and resident there (upload() only
        records a stream): the same plan Plan.from_slices builds for the same slices and
        tile sizes (bsfa_plan_from_dcsr)."""
        h = ctypes.c_void_p()
        _check("bsfa_plan_from_dcsr", library().bsfa_plan_from_dcsr(self._h, hq, hkv, d, ctypes.byref(h)))
        return Plan(h)

    def close(self):
        if self._h is not None and self._h.value:
            library().bsfa_dcsr_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Plan:
    """A compiled mask (tile CSR + pieces) with its schedule.  Host-only until upload()."""

    def __init__(self, handle):
        self._h = handle
        self._info = None

    # -- constructors ---------------------------------------------------------
    @classmethod
    def from_slices(cls, slices, sq, sk, hq, hkv, d, bq=128, bk=128):
        arr = slice_array(slices)
        h = ctypes.c_void_p()
        _check("bsfa_plan_create", library().bsfa_plan_create(_ptr(arr), len(arr), sq, sk, hq, hkv, d,
                                                               bq, bk, ctypes.byref(h)))
        return cls(h)

    @classmethod
    def from_varlen(cls, cu_seqlens, hq, hkv, d, causal=True, bq=128, bk=128):
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        h = ctypes.c_void_p()
        _check("bsfa_plan_from_varlen", library().bsfa_plan_from_varlen(
            _ptr(cu), len(cu) - 1, 1 if causal else 0, hq, hkv, d, bq, bk, ctypes.byref(h)))
        return cls(h)

    @classmethod
    def from_blocks(cls, codes, block_q, block_k, sq, sk, hq, hkv, d, bq=128, bk=128):
        c = np.ascontiguousarray(codes, dtype=np.uint8)
        h = ctypes.c_void_p()
        _check("bsfa_plan_from_blocks", library().bsfa_plan_from_blocks(
            _ptr(c), c.shape[0], c.shape[1], block_q, block_k, sq, sk, hq, hkv, d, bq, bk,
            ctypes.byref(h)))
        return cls(h)

    # -- lifecycle ------------------------------------------------------------
    def upload(self, stream=None):
        _check("bsfa_plan_upload", library().bsfa_plan_upload(self._h, _stream_handle(stream)))
        return self

    def close(self):
        if self._h is not None and self._h.value:
            library().bsfa_plan_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    # -- inspection -----------------------------------------------------------
    def info(self) -> dict:
        """Plan statistics; shapes and counts are fixed at creation, so they are cached."""
        inf = PlanInfo()
        _check("bsfa_plan_get_info", library().bsfa_plan_get_info(self._h, ctypes.byref(inf)))
        d = {name: getattr(inf, name) for name, _ in PlanInfo._fields_}
        self._info = d
        return d

    def shapes(self):
        """(sq, sk, hq, hkv, d) of the plan."""
        if self._info is None:
            self.info()
        i = self._info
        return i["sq"], i["sk"], i["hq"], i["hkv"], i["d"]

    def pieces(self):
        """(piece_ptr [nnz + 1], pieces [n_pieces, 5]) of the host compiler."""
        inf = self.info()
        piece_ptr = np.zeros(inf["nnz"] + 1, np.int32)
        pieces = np.zeros((max(1, inf["n_pieces"]), 5), np.int32)
        _check("bsfa_plan_export_pieces", library().bsfa_plan_export_pieces(
            self._h, _ptr(piece_ptr), _ptr(pieces), inf["n_pieces"]))
        return piece_ptr, pieces[:inf["n_pieces"]]

    def csr(self):
        inf = self.info()
        row_ptr = np.zeros(inf["n_qtiles"] + 1, np.int32)
        nnz = inf["nnz"]
        col = np.zeros(max(1, nnz), np.int32)
        tag = np.zeros(max(1, nnz), np.uint8)
        n = ctypes.c_int64(0)
        _check("bsfa_plan_export_csr", library().bsfa_plan_export_csr(
            self._h, _ptr(row_ptr), _ptr(col), _ptr(tag), len(col), ctypes.byref(n)))
        return row_ptr, col[:n.value].copy(), tag[:n.value].copy()

    def schedule(self):
        """(bin_ptr [n_bins + 1], unit ids in execution order [n_units], unit cost by unit id).
        Without split rows, unit id == item id == h * n_qtiles + qtile."""
        inf = self.info()
        bin_ptr = np.zeros(inf["n_bins"] + 1, np.int32)
        units = np.zeros(max(1, inf["n_units"]), np.int32)
        cost = np.zeros(max(1, inf["n_units"]), np.float32)
        _check("bsfa_plan_export_schedule", library().bsfa_plan_export_schedule(
            self._h, _ptr(bin_ptr), _ptr(units), _ptr(cost)))
        return bin_ptr, units[:inf["n_units"]], cost[:inf["n_units"]]

    def units(self):
        """[n_units, 4] int32: item, first entry, end entry (CSR indices), partial slot or -1."""
        inf = self.info()
        u = np.zeros((max(1, inf["n_units"]), 4), np.int32)
        _check("bsfa_plan_export_units", library().bsfa_plan_export_units(self._h, _ptr(u)))
        return u[:inf["n_units"]]


def to_device_bf16(bits: np.ndarray, device="cuda"):
    """Seeded bf16 bit patterns (uint16 numpy) -> a bf16 device tensor of the same shape."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def _tview(t):
    """bsfa_tensor for a [tokens, heads, d] torch tensor with contiguous last dim."""
    assert t.dim() == 3 and t.stride(2) == 1, "expected [tokens, heads, d] with d contiguous"
    return Tensor(ctypes.c_void_p(t.data_ptr()), t.stride(0), t.stride(1))


def workspace_for(plan: Plan, device="cuda"):
    """Device workspace for the split rows of a plan (None when no row is split)."""
    import torch
    n = plan.info()["workspace_bytes"]
    if n == 0:
        return None
    return torch.empty(n // 4, dtype=torch.float32, device=device)


def _on_device(**named):
    """The library hands these addresses to the GPU as they are: each tensor must live on
    the current CUDA device (a host tensor's address would reach a kernel)."""
    import torch
    dev = torch.cuda.current_device() if torch.cuda.is_available() else None
    for name, t in named.items():
        if t is not None and (not t.is_cuda or t.device.index != dev):
            raise ValueError(f"{name} must be a CUDA tensor on the current device "
                             f"(cuda:{dev}), got one on {t.device}")


DTYPE_BF16, DTYPE_F32 = 0, 1   # element types of O for the typed entry points


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise ValueError(f"O must be bf16 or fp32, got {t.dtype}")


def attn_fwd(q, k, v, plan: Plan, scale: float, out=None, lse=None, workspace=None, stream=None,
             out_dtype=None):
    """Forward over the plan's mask.  q [sq, hq, d], k/v [sk, hkv, d] bf16 CUDA tensors.
    workspace: fp32 device tensor of at least the plan's workspace_bytes when a row is
    split (allocated here when not given).  O is bf16 unless `out` is an fp32 tensor or
    out_dtype is torch.float32 (the fp32 value the bf16 output is rounded from).

    Returns (O [sq, hq, d], LSE [hq, sq] fp32)."""
    import torch
    sq, hq, d = q.shape
    psq, psk, phq, phkv, pd = plan.shapes()
    if (sq, hq, d) != (psq, phq, pd):
        raise ValueError(f"q shape {tuple(q.shape)} does not match the plan ({psq}, {phq}, {pd})")
    for name, t in (("k", k), ("v", v)):
        if tuple(t.shape) != (psk, phkv, pd):
            raise ValueError(f"{name} shape {tuple(t.shape)} does not match the plan "
                             f"({psk}, {phkv}, {pd})")
    if out is None:
        out = torch.empty((sq, hq, d), dtype=out_dtype or torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((hq, sq), dtype=torch.float32, device=q.device)
    assert q.dtype == k.dtype == v.dtype == torch.bfloat16
    o_code = _dtype_code(out)
    assert out_dtype is None or out.dtype == out_dtype
    assert tuple(out.shape) == (sq, hq, d)
    assert lse.dtype == torch.float32 and lse.stride(1) == 1 and lse.shape[0] == hq
    if lse.shape[1] < sq:
        raise ValueError(f"lse covers {lse.shape[1]} tokens, fewer than the {sq} queries")
    _on_device(q=q, k=k, v=v, out=out, lse=lse, workspace=workspace)
    if workspace is None and plan.info()["workspace_bytes"] > 0:
        workspace = workspace_for(plan, q.device)
        if stream is not None:
            # allocated on the current stream, used on `stream`: keep the allocator from
            # handing the memory out again before that stream's work has run
            workspace.record_stream(stream)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                            workspace.numel() * workspace.element_size())
    tq, tk, tv, to = _tview(q), _tview(k), _tview(v), _tview(out)
    if o_code == DTYPE_BF16:
        _check("bsfa_attn_fwd", library().bsfa_attn_fwd(
            ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), plan.handle, float(scale),
            ctypes.byref(to), ctypes.c_void_p(lse.data_ptr()), lse.stride(0), ctypes.c_void_p(ws_ptr),
            ws_bytes, _stream_handle(stream)))
    else:
        _check("bsfa_attn_fwd_typed", library().bsfa_attn_fwd_typed(
            ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), plan.handle, float(scale),
            ctypes.byref(to), o_code, ctypes.c_void_p(lse.data_ptr()), lse.stride(0), ctypes.c_void_p(ws_ptr),
            ws_bytes, _stream_handle(stream)))
    return out, lse


def attn_bwd(q, k, v, dout, lse, plan: Plan, scale: float, dq=None, dk=None, dv=None,
             delta=None, stream=None, o=None):
    """Gradients of the plan's masked attention.  q/dout [sq, hq, d], k/v [sk, hkv, d]
    bf16; lse [hq, >= sq] fp32 from the forward.  o: the forward's fp32 output
    (attn_fwd(..., out_dtype=torch.float32)), optional: with it D_i = dO_i . O_i comes from
    O and the separate D pass is skipped.

    Returns (dQ [sq, hq, d], dK [sk, hkv, d], dV [sk, hkv, d]) fp32; delta (D_i =
    sum_j P_ij dP_ij, shaped like lse) is scratch the call fills."""
    import torch
    sq, hq, d = q.shape
    psq, psk, phq, phkv, pd = plan.shapes()
    if (sq, hq, d) != (psq, phq, pd):
        raise ValueError(f"q shape {tuple(q.shape)} does not match the plan ({psq}, {phq}, {pd})")
    for name, t, shp in (("k", k, (psk, phkv, pd)), ("v", v, (psk, phkv, pd)),
                         ("dout", dout, (psq, phq, pd))):
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} shape {tuple(t.shape)} does not match the plan {shp}")
        assert t.dtype == torch.bfloat16, f"{name} must be bf16"
    assert q.dtype == torch.bfloat16
    assert lse.dtype == torch.float32 and lse.stride(1) == 1 and lse.shape[0] == hq
    if lse.shape[1] < sq:
        raise ValueError(f"lse covers {lse.shape[1]} tokens, fewer than the {sq} queries")
    _on_device(q=q, k=k, v=v, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta, o=o)
    dev = q.device
    if dq is None:
        dq = torch.empty((sq, hq, d), dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.empty((psk, phkv, d), dtype=torch.float32, device=dev)
    if dv is None:
        dv = torch.empty((psk, phkv, d), dtype=torch.float32, device=dev)
    if delta is None:
        delta = torch.empty_like(lse)
    for name, t, shp in (("dq", dq, (sq, hq, d)), ("dk", dk, (psk, phkv, d)), ("dv", dv, (psk, phkv, d))):
        assert t.dtype == torch.float32 and t.is_contiguous() and tuple(t.shape) == shp, name
    assert delta.dtype == torch.float32 and delta.stride() == lse.stride() and delta.shape == lse.shape
    tq, tk, tv, tg = _tview(q), _tview(k), _tview(v), _tview(dout)
    if o is None:
        _check("bsfa_attn_bwd", library().bsfa_attn_bwd(
            ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), ctypes.byref(tg),
            ctypes.c_void_p(lse.data_ptr()), lse.stride(0), plan.handle, float(scale),
            ctypes.c_void_p(dq.data_ptr()), ctypes.c_void_p(dk.data_ptr()), ctypes.c_void_p(dv.data_ptr()),
            ctypes.c_void_p(delta.data_ptr()), _stream_handle(stream)))
        return dq, dk, dv
    if o.dtype != torch.float32:
        raise ValueError("o must be the forward's fp32 output (attn_fwd(..., out_dtype=torch.float32))")
    if tuple(o.shape) != (sq, hq, d):
        raise ValueError(f"o shape {tuple(o.shape)} does not match the plan ({sq}, {hq}, {d})")
    to = _tview(o)
    _check("bsfa_attn_bwd_o32", library().bsfa_attn_bwd_o32(
        ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), ctypes.byref(tg), ctypes.byref(to),
        ctypes.c_void_p(lse.data_ptr()), lse.stride(0), plan.handle, float(scale),
        ctypes.c_void_p(dq.data_ptr()), ctypes.c_void_p(dk.data_ptr()), ctypes.c_void_p(dv.data_ptr()),
        ctypes.c_void_p(delta.data_ptr()), _stream_handle(stream)))
    return dq, dk, dv


def attn_merge(o_parts, lse_parts, out=None, lse=None, stream=None, out_dtype=None):
    """Merge n partials: o_parts list of [T, H, d] tensors of one dtype, bf16 or fp32 (same
    strides), lse_parts list of [H, T] fp32.  The result O is bf16 unless `out` is fp32 or
    out_dtype is torch.float32."""
    import torch
    n = len(o_parts)
    assert n == len(lse_parts) and n >= 1
    t, h, d = o_parts[0].shape
    st = o_parts[0].stride()
    if st[2] != 1:
        raise ValueError("partials need a contiguous head dim (stride 1)")
    p_code = _dtype_code(o_parts[0])
    for p in o_parts:
        assert p.shape == (t, h, d) and p.stride() == st and p.dtype == o_parts[0].dtype
    lst = lse_parts[0].stride(0)
    for l in lse_parts:
        assert l.shape[0] == h and l.stride(0) == lst and l.stride(1) == 1 and l.dtype == torch.float32
        if l.shape[1] < t:
            raise ValueError(f"an LSE part covers {l.shape[1]} tokens, fewer than the {t} merged")
    if out is None:
        out = torch.empty((t, h, d), dtype=out_dtype or torch.bfloat16, device=o_parts[0].device)
    o_code = _dtype_code(out)
    assert out_dtype is None or out.dtype == out_dtype
    if tuple(out.shape) != (t, h, d):
        raise ValueError(f"out shape {tuple(out.shape)} does not match the partials ({t}, {h}, {d})")
    if lse is None:
        lse = torch.empty((h, lst), dtype=torch.float32, device=o_parts[0].device)
    if lse.dtype != torch.float32 or lse.dim() != 2 or lse.shape[0] != h or lse.shape[1] < t \
            or lse.stride(1) != 1:
        raise ValueError(f"lse must be fp32 [{h}, >= {t}] with contiguous tokens, got "
                         f"{lse.dtype} {tuple(lse.shape)}")
    assert lse.stride(0) == lst
    _on_device(**{f"o_parts[{i}]": p for i, p in enumerate(o_parts)},
               **{f"lse_parts[{i}]": l for i, l in enumerate(lse_parts)}, out=out, lse=lse)
    optrs = (ctypes.c_void_p * n)(*[p.data_ptr() for p in o_parts])
    lptrs = (ctypes.c_void_p * n)(*[l.data_ptr() for l in lse_parts])
    to = _tview(out)
    if p_code == DTYPE_BF16 and o_code == DTYPE_BF16:
        _check("bsfa_attn_merge", library().bsfa_attn_merge(
            optrs, lptrs, n, st[0], st[1], lst, t, h, d, ctypes.byref(to),
            ctypes.c_void_p(lse.data_ptr()), _stream_handle(stream)))
    else:
        _check("bsfa_attn_merge_typed", library().bsfa_attn_merge_typed(
            optrs, p_code, lptrs, n, st[0], st[1], lst, t, h, d, ctypes.byref(to), o_code,
            ctypes.c_void_p(lse.data_ptr()), _stream_handle(stream)))
    return out, lse[:, :t]


def set_rescale_threshold(tau_log2: float):
    """Conditional-rescale threshold of the forward (log2 units, default 8; process-wide)."""
    _check("bsfa_set_rescale_threshold", library().bsfa_set_rescale_threshold(float(tau_log2)))


def rescale_threshold() -> float:
    return float(library().bsfa_get_rescale_threshold())


def lpt_assign(costs, n_bins):
    """Scheduler core on an explicit cost list: (bin_of int32 [n], bin_load [n_bins], makespan)."""
    c = np.ascontiguousarray(costs, dtype=np.float32)
    bin_of = np.zeros(max(1, len(c)), np.int32)
    load = np.zeros(max(1, n_bins), np.float64)
    mk = library().bsfa_lpt_assign(_ptr(c), len(c), n_bins, _ptr(bin_of), _ptr(load))
    if mk < 0:
        raise BsfaError("bsfa_lpt_assign", 1)
    return bin_of[:len(c)], load[:n_bins], mk


def plan_from_workload(w, bq=128, bk=128, upload=True, stream=None) -> Plan:
    """Plan for a workloads.Workload using its native mask form (varlen, blocks or slices)."""
    if w.cu_seqlens is not None:
        p = Plan.from_varlen(w.cu_seqlens, w.hq, w.hkv, w.d, causal=True, bq=bq, bk=bk)
    elif w.block_codes is not None:
        p = Plan.from_blocks(w.block_codes, w.block[0], w.block[1], w.sq, w.sk, w.hq, w.hkv, w.d,
                             bq=bq, bk=bk)
    else:
        p = Plan.from_slices(w.slices, w.sq, w.sk, w.hq, w.hkv, w.d, bq=bq, bk=bk)
    if upload:
        p.upload(stream)
    return p
