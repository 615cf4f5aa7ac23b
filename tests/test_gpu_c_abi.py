"""The C ABI from a C99 program (tests/c_abi/abi_forward.c, built by build()): no Python
binding and no torch in the process that calls the library.  The inputs come from the
seeded generators; the program writes O and LSE, which are compared with the oracle."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from block_sparse_flash_csr_amd import workloads as W

from gpu_helpers import compare, say

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "abi_forward")


@pytest.mark.parametrize("seed,lengths,hq,hkv,d", [
    (71, [300, 129, 271], 4, 2, 128),
    (72, [64, 700, 1, 200], 3, 1, 64),
])
def test_c_program_forward_matches_oracle(tmp_path, seed, lengths, hq, hkv, d):
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: run build() first")
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    s = int(cu[-1])
    qb, kb, vb = W.random_inputs(rng, s, s, hq, hkv, d)
    scale = 1.0 / np.sqrt(d)
    with open(tmp_path / "case.txt", "w") as f:
        f.write(f"{s} {hq} {hkv} {d} {len(lengths)} {float(scale)!r}\n" + " ".join(str(int(x)) for x in cu) + "\n")
    for name, a in (("q", qb), ("k", kb), ("v", vb)):
        np.ascontiguousarray(a, dtype=np.uint16).tofile(tmp_path / f"{name}.bin")
    say(f"C program forward: seed={seed} docs={lengths} hq={hq} hkv={hkv} d={d}")
    r = subprocess.run([EXE, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    say(r.stdout.strip())
    o = np.fromfile(tmp_path / "o.bin", dtype=np.uint16).reshape(s, hq, d)
    lse = np.fromfile(tmp_path / "lse.bin", dtype=np.float32).reshape(hq, s)
    slices = [(int(cu[t]), int(cu[t + 1]), int(cu[t]), int(cu[t + 1]), 1) for t in range(len(lengths))]
    o_ref, lse_ref = oracle.attn_fwd(qb, kb, vb, slices, scale)
    compare(W.bf16_to_f32(o), lse.T, o_ref, lse_ref.T, f"C program seed={seed}")
