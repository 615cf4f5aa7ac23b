"""Mask compiler (library) against the CSR oracle: bit-exact row_ptr / col / tag on the
five workloads and on random small slice lists; exact pair counts."""
import numpy as np
import pytest

import oracle
from block_sparse_flash_csr_amd import api
from block_sparse_flash_csr_amd import workloads as W


def _compare(plan, slices, sq, sk, bq, bk):
    rp, col, tag = plan.csr()
    rp2, col2, tag2 = oracle.tile_csr(slices, sq, sk, bq, bk)
    assert np.array_equal(rp, rp2)
    assert np.array_equal(col, col2)
    assert np.array_equal(tag, tag2)
    assert plan.info()["pairs"] == oracle.pair_count(slices, sq)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_workload_csr_bit_exact(cfg):
    w = W.WORKLOADS[cfg](with_inputs=False)
    plan = api.plan_from_workload(w, upload=False)
    _compare(plan, w.slices, w.sq, w.sk, 128, 128)
    # the slice form of the same mask compiles to the same CSR
    plan2 = api.Plan.from_slices(w.slices, w.sq, w.sk, w.hq, w.hkv, w.d)
    r1, c1, t1 = plan.csr()
    r2, c2, t2 = plan2.csr()
    assert np.array_equal(r1, r2) and np.array_equal(c1, c2) and np.array_equal(t1, t2)


def test_workload5_chunks_bit_exact():
    w = W.kv_split_q8192(with_inputs=False)
    c = w.extra["chunk"]
    for sl in w.extra["chunk_slices"]:
        plan = api.Plan.from_slices(sl, c, c, w.hq, w.hkv, w.d)
        _compare(plan, sl, c, c, 128, 128)
    # the unsplit mask against all 8 chunks at once
    plan = api.Plan.from_slices(w.slices, w.sq, w.sk, w.hq, w.hkv, w.d)
    _compare(plan, w.slices, w.sq, w.sk, 128, 128)


def test_workload_tile_counts():
    expect = {1: (1, 2), 2: (1135, 358), 3: (4192, 256), 4: (52496, 736)}
    for cfg, (nf, npart) in expect.items():
        w = W.WORKLOADS[cfg](with_inputs=False)
        inf = api.plan_from_workload(w, upload=False).info()
        assert (inf["n_full"], inf["n_partial"]) == (nf, npart), cfg


@pytest.mark.parametrize("bq,bk", [(16, 16), (16, 32), (32, 16), (32, 64), (64, 128), (128, 128),
                                   (128, 64), (7, 13)])
def test_random_masks_bit_exact(bq, bk):
    rng = np.random.default_rng(bq * 1000 + bk)
    for _ in range(25):
        sq, sk = int(rng.integers(1, 520)), int(rng.integers(1, 520))
        slices = W.random_slices(rng, sq, sk, int(rng.integers(0, 9)))
        plan = api.Plan.from_slices(slices, sq, sk, 2, 1, 64, bq=bq, bk=bk)
        _compare(plan, slices, sq, sk, bq, bk)


def test_union_of_partial_slices_is_full():
    """Two slices that each cover part of a tile but together cover all of it: tag full."""
    slices = [(0, 128, 0, 50, 0), (0, 128, 50, 128, 0)]
    plan = api.Plan.from_slices(slices, 128, 128, 1, 1, 128)
    _, col, tag = plan.csr()
    assert list(col) == [0] and list(tag) == [1]
    # a causal slice plus the full rectangle above its diagonal: full as well
    slices = [(0, 128, 0, 128, 1), (0, 128, 0, 128, 0)]
    _, col, tag = api.Plan.from_slices(slices, 128, 128, 1, 1, 128).csr()
    assert list(tag) == [1]


def test_empty_mask_and_empty_rows():
    plan = api.Plan.from_slices([], 300, 200, 1, 1, 128)
    rp, col, tag = plan.csr()
    assert np.all(rp == 0) and len(col) == 0
    assert plan.info()["pairs"] == 0
    # rows 128..255 empty
    slices = [(0, 100, 0, 200, 0), (260, 300, 0, 10, 0)]
    _compare(api.Plan.from_slices(slices, 300, 200, 1, 1, 128), slices, 300, 200, 128, 128)


def test_blocks_and_varlen_forms_match_slices():
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 3, size=(5, 7)).astype(np.uint8)
    sq, sk = 5 * 48 - 10, 7 * 40 - 3
    plan = api.Plan.from_blocks(codes, 48, 40, sq, sk, 2, 2, 64)
    slices = W.block_slices(codes, 48, 40, sq, sk)
    _compare(plan, slices, sq, sk, 128, 128)
    cu = np.array([0, 5, 5, 300, 301, 777], np.int32)
    for causal in (True, False):
        plan = api.Plan.from_varlen(cu, 4, 2, 64, causal=causal)
        sl = [(int(cu[i]), int(cu[i + 1]), int(cu[i]), int(cu[i + 1]), 1 if causal else 0)
              for i in range(len(cu) - 1) if cu[i + 1] > cu[i]]
        _compare(plan, sl, 777, 777, 128, 128)


def _piece_mask(pieces, r0, r1, c0, c1):
    m = np.zeros((r1 - r0, c1 - c0), bool)
    for q_lo, q_hi, k_lo, k_hi, diag in pieces:
        for i in range(q_lo, q_hi):
            hi = min(k_hi, i + diag + 1)
            if k_lo < hi:
                m[i - r0, k_lo - c0:hi - c0] = True
    return m


@pytest.mark.parametrize("bq,bk", [(16, 16), (32, 64), (128, 128), (7, 13)])
def test_pieces_reproduce_the_mask_of_partial_tiles(bq, bk):
    """Inside every partial tile the union of its stored pieces admits exactly the pairs
    of the oracle's row key sets (and every full tile admits all of its pairs)."""
    rng = np.random.default_rng(7 * bq + bk)
    for _ in range(6):
        sq, sk = int(rng.integers(1, 300)), int(rng.integers(1, 300))
        slices = W.random_slices(rng, sq, sk, int(rng.integers(1, 7)))
        plan = api.Plan.from_slices(slices, sq, sk, 1, 1, 64, bq=bq, bk=bk)
        rp, col, tag = plan.csr()
        pp, pcs = plan.pieces()
        dense = np.zeros((sq, sk), bool)
        for i in range(sq):
            for lo, hi in oracle.row_key_set(slices, i):
                dense[i, lo:hi] = True
        for qt in range(len(rp) - 1):
            r0, r1 = qt * bq, min(qt * bq + bq, sq)
            for e in range(rp[qt], rp[qt + 1]):
                c0, c1 = col[e] * bk, min(col[e] * bk + bk, sk)
                want = dense[r0:r1, c0:c1]
                if tag[e] == 1:
                    assert want.all() and pp[e] == pp[e + 1]
                else:
                    got = _piece_mask(pcs[pp[e]:pp[e + 1]], r0, r1, c0, c1)
                    assert np.array_equal(got, want), (qt, col[e])
