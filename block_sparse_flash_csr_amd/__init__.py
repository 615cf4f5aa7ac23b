"""block_sparse_flash_csr_amd: masked flash-attention forward, its backward and the KV-partial merge for
gfx950 behind a C-ABI library (libbsfa.so).  The API objects load the library lazily."""
from __future__ import annotations


def __getattr__(name):
    if name in ("Plan", "DeviceCsr", "attn_fwd", "attn_bwd", "attn_merge", "BsfaError", "library", "plan_from_workload"):
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
