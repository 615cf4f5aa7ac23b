"""Pins of the fp64 oracle against facts that do not come from the oracle itself:
brute force on tiny inputs (explicit dense masks + scipy's logsumexp), closed
forms, invariants of the KV-split merge, closed-form pair and tile counts, and
the worked values printed on the pages (tests/golden/)."""
import json
import os

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from block_sparse_flash_csr_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# Independent brute force: a dense boolean mask built pair by pair from the
# slice definitions, dense fp64 scores, scipy logsumexp.
# --------------------------------------------------------------------------
def dense_mask(slices, sq, sk):
    m = np.zeros((sq, sk), bool)
    for (q0, q1, k0, k1, t) in slices:
        for i in range(max(q0, 0), min(q1, sq)):
            for j in range(max(k0, 0), min(k1, sk)):
                if t == W.FULL or (j - k1 <= i - q1):
                    m[i, j] = True
    return m


def brute_attention(qb, kb, vb, slices, scale):
    q = W.bf16_to_f32(qb).astype(np.float64)
    k = W.bf16_to_f32(kb).astype(np.float64)
    v = W.bf16_to_f32(vb).astype(np.float64)
    sq, hq, d = q.shape
    sk, hkv, _ = k.shape
    mask = dense_mask(slices, sq, sk)
    o = np.zeros((sq, hq, d))
    lse = np.full((hq, sq), -np.inf)
    for h in range(hq):
        g = h // (hq // hkv)
        s = scale * (q[:, h, :] @ k[:, g, :].T)
        for i in range(sq):
            js = np.nonzero(mask[i])[0]
            if js.size == 0:
                continue
            lse[h, i] = logsumexp(s[i, js])
            o[i, h] = np.exp(s[i, js] - lse[h, i]) @ v[js, g, :]
    return o, lse


def _inputs(seed, sq, sk, hq, hkv, d):
    rng = np.random.default_rng(seed)
    return W.random_inputs(rng, sq, sk, hq, hkv, d)


CASES = [
    # (seed, sq, sk, hq, hkv, d, n_slices)
    (11, 37, 37, 2, 2, 16, 3),
    (12, 64, 48, 4, 2, 8, 5),
    (13, 29, 61, 3, 1, 16, 4),
    (14, 50, 50, 2, 1, 4, 1),
    (15, 17, 9, 1, 1, 16, 6),
]


@pytest.mark.parametrize("case", CASES)
def test_brute_force_tiny(case):
    seed, sq, sk, hq, hkv, d, n = case
    rng = np.random.default_rng(seed + 1000)
    slices = W.random_slices(rng, sq, sk, n)
    qb, kb, vb = _inputs(seed, sq, sk, hq, hkv, d)
    scale = 1.0 / np.sqrt(d)
    o_ref, lse_ref = brute_attention(qb, kb, vb, slices, scale)
    o, lse = oracle.attn_fwd(qb, kb, vb, slices, scale, n_threads=2)
    assert np.array_equal(np.isinf(lse), np.isinf(lse_ref))
    fin = np.isfinite(lse_ref)
    np.testing.assert_allclose(lse[fin], lse_ref[fin], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    # empty rows: exact zeros
    for h in range(hq):
        rows = np.nonzero(~fin[h])[0]
        assert np.all(o[rows, h, :] == 0.0)


def test_brute_force_causal_alignments():
    """Bottom-right causal with |q| != |k| in both directions, and the usual square case."""
    sq, sk, d = 24, 40, 8
    qb, kb, vb = _inputs(21, sq, sk, 1, 1, d)
    for slices in ([(0, 24, 0, 40, W.CAUSAL)], [(4, 20, 30, 38, W.CAUSAL)],
                   [(0, 24, 10, 14, W.CAUSAL), (0, 24, 0, 24, W.CAUSAL)]):
        o_ref, lse_ref = brute_attention(qb, kb, vb, slices, 0.3)
        o, lse = oracle.attn_fwd(qb, kb, vb, slices, 0.3, n_threads=1)
        np.testing.assert_allclose(o, o_ref, atol=1e-12)
        fin = np.isfinite(lse_ref)
        assert np.array_equal(fin, np.isfinite(lse))
        np.testing.assert_allclose(lse[fin], lse_ref[fin], atol=1e-12)


def test_row_key_set_is_union():
    rng = np.random.default_rng(5)
    for trial in range(20):
        sq, sk = 33, 47
        slices = W.random_slices(rng, sq, sk, int(rng.integers(1, 7)))
        mask = dense_mask(slices, sq, sk)
        for i in range(sq):
            ivs = oracle.row_key_set(slices, i)
            got = np.zeros(sk, bool)
            prev_hi = -1
            for lo, hi in ivs:
                assert lo > prev_hi, "intervals must be sorted, disjoint and non-touching"
                prev_hi = hi
                got[lo:hi] = True
            assert np.array_equal(got, mask[i])


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------
def test_zero_query_gives_mean_of_values():
    sq, sk, d = 31, 31, 16
    rng = np.random.default_rng(7)
    slices = W.random_slices(rng, sq, sk, 4)
    _, kb, vb = _inputs(8, sq, sk, 1, 1, d)
    qb = np.zeros((sq, 1, d), np.uint16)
    o, lse = oracle.attn_fwd(qb, kb, vb, slices, 0.7, n_threads=1)
    v = W.bf16_to_f32(vb).astype(np.float64)[:, 0, :]
    mask = dense_mask(slices, sq, sk)
    for i in range(sq):
        n = mask[i].sum()
        if n == 0:
            assert lse[0, i] == -np.inf and np.all(o[i, 0] == 0)
        else:
            assert abs(lse[0, i] - np.log(n)) < 1e-12
            np.testing.assert_allclose(o[i, 0], v[mask[i]].mean(axis=0), atol=1e-12)


def test_single_key_rows():
    """Row i sees exactly key i: O = v_i, LSE = s_ii."""
    s, d = 20, 16
    slices = [(i, i + 1, i, i + 1, W.FULL) for i in range(s)]
    qb, kb, vb = _inputs(9, s, s, 2, 2, d)
    o, lse = oracle.attn_fwd(qb, kb, vb, slices, 0.25, n_threads=1)
    q = W.bf16_to_f32(qb).astype(np.float64)
    k = W.bf16_to_f32(kb).astype(np.float64)
    v = W.bf16_to_f32(vb).astype(np.float64)
    for h in range(2):
        for i in range(s):
            assert np.array_equal(o[i, h], v[i, h])
            assert abs(lse[h, i] - 0.25 * float(q[i, h] @ k[i, h])) < 1e-12


def test_constant_values():
    s, d = 40, 8
    rng = np.random.default_rng(10)
    slices = W.random_slices(rng, s, s, 5)
    qb, kb, _ = _inputs(10, s, s, 1, 1, d)
    vb = np.full((s, 1, d), W.bf16_bits(np.array([1.75], np.float32))[0], np.uint16)
    o, lse = oracle.attn_fwd(qb, kb, vb, slices, 0.5, n_threads=1)
    fin = np.isfinite(lse[0])
    np.testing.assert_allclose(o[fin, 0], 1.75, atol=1e-12)
    assert np.all(o[~fin, 0] == 0)


def test_one_hot_values_give_probabilities():
    """S_k <= d and V = identity rows: O row i = softmax row i, which sums to 1."""
    sq, sk, d = 24, 16, 16
    rng = np.random.default_rng(11)
    slices = W.random_slices(rng, sq, sk, 3, allow_empty=False)
    qb, kb, _ = _inputs(11, sq, sk, 1, 1, d)
    eye = np.eye(sk, d, dtype=np.float32)[:, None, :]
    vb = W.bf16_bits(eye)
    o, lse = oracle.attn_fwd(qb, kb, vb, slices, 1.0, n_threads=1)
    mask = dense_mask(slices, sq, sk)
    for i in range(sq):
        p = o[i, 0, :sk]
        if mask[i].any():
            assert abs(p.sum() - 1.0) < 1e-12
            assert np.all(p[~mask[i]] == 0) and np.all(p[mask[i]] > 0)
        else:
            assert np.all(p == 0)


# --------------------------------------------------------------------------
# Masked entries contribute nothing (bitwise)
# --------------------------------------------------------------------------
def test_masked_perturbation_is_bitwise_invisible():
    s, d = 48, 16
    slices = [(0, 24, 0, 24, W.CAUSAL), (24, 48, 8, 40, W.FULL)]
    qb, kb, vb = _inputs(12, s, s, 2, 1, d)
    o0, l0 = oracle.attn_fwd(qb, kb, vb, slices, 0.3, n_threads=2)
    kb2, vb2 = kb.copy(), vb.copy()
    big = W.bf16_bits(np.array([3.0e4], np.float32))[0]
    kb2[40:] = big      # keys >= 40 are masked for every row
    vb2[40:] = big
    kb2[24:40, :, ::2] = big  # keys 24..39 are masked for rows 0..23
    vb2[24:40] = big
    o1, l1 = oracle.attn_fwd(qb, kb2, vb2, slices, 0.3, n_threads=2)
    assert np.array_equal(o0[:24], o1[:24]) and np.array_equal(l0[:, :24], l1[:, :24])


# --------------------------------------------------------------------------
# KV split and merge
# --------------------------------------------------------------------------
def split_slices(slices, c0, c1):
    """The part of a slice mask with keys in [c0, c1), in chunk-local key coordinates.
    A causal slice clipped on its right edge keeps its diagonal: rows past the
    clipped corner become full."""
    out = []
    for (q0, q1, k0, k1, t) in slices:
        a, b = max(k0, c0), min(k1, c1)
        if a >= b or q0 >= q1:
            continue
        if t == W.FULL:
            out.append((q0, q1, a - c0, b - c0, W.FULL))
            continue
        shift = k1 - b              # rows i >= q1 - shift see every key up to b
        qc = q1 - shift
        if qc > q0:
            out.append((q0, qc, a - c0, b - c0, W.CAUSAL))
        if qc < q1:
            out.append((max(q0, qc), q1, a - c0, b - c0, W.FULL))
    return out


def test_split_slices_helper_matches_dense_mask():
    rng = np.random.default_rng(13)
    for _ in range(30):
        sq, sk = 30, 50
        slices = W.random_slices(rng, sq, sk, 4)
        full = dense_mask(slices, sq, sk)
        cuts = sorted(set([0, sk] + list(rng.integers(1, sk, size=3))))
        for c0, c1 in zip(cuts[:-1], cuts[1:]):
            part = dense_mask(split_slices(slices, c0, c1), sq, c1 - c0)
            assert np.array_equal(part, full[:, c0:c1])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_split_then_merge_equals_unsplit(seed):
    rng = np.random.default_rng(100 + seed)
    sq, sk, hq, hkv, d = 40, 70, 4, 2, 16
    slices = W.random_slices(rng, sq, sk, 5)
    qb, kb, vb = _inputs(200 + seed, sq, sk, hq, hkv, d)
    o_ref, lse_ref = oracle.attn_fwd(qb, kb, vb, slices, 0.4, n_threads=2)
    cuts = [0, 13, 29, 30, 55, 70]
    parts_o, parts_l = [], []
    for c0, c1 in zip(cuts[:-1], cuts[1:]):
        o, l = oracle.attn_fwd(qb, kb[c0:c1], vb[c0:c1], split_slices(slices, c0, c1), 0.4,
                               n_threads=2)
        parts_o.append(o.transpose(1, 0, 2).reshape(hq * sq, d))
        parts_l.append(l.reshape(hq * sq))
    po, pl = np.stack(parts_o), np.stack(parts_l)
    om, lm = oracle.merge(po, pl)
    fin = np.isfinite(lse_ref.reshape(-1))
    assert np.array_equal(fin, np.isfinite(lm))
    np.testing.assert_allclose(lm[fin], lse_ref.reshape(-1)[fin], atol=1e-12)
    np.testing.assert_allclose(om, o_ref.transpose(1, 0, 2).reshape(hq * sq, d), atol=1e-12)
    # order invariance
    perm = [3, 0, 4, 2, 1]
    om2, lm2 = oracle.merge(po[perm], pl[perm])
    np.testing.assert_allclose(om2, om, atol=1e-13)
    np.testing.assert_allclose(lm2[fin], lm[fin], atol=1e-13)


def test_merge_closed_forms():
    rng = np.random.default_rng(3)
    r, d = 16, 8
    o1 = rng.standard_normal((r, d))
    o2 = rng.standard_normal((r, d))
    a = rng.standard_normal(r)
    # equal LSE: the average, LSE + ln 2
    om, lm = oracle.merge(np.stack([o1, o2]), np.stack([a, a]))
    np.testing.assert_allclose(om, 0.5 * (o1 + o2), atol=1e-14)
    np.testing.assert_allclose(lm, a + np.log(2.0), atol=1e-14)
    # a partial at -inf is the identity
    om, lm = oracle.merge(np.stack([o1, o2 * 0]), np.stack([a, np.full(r, -np.inf)]))
    np.testing.assert_allclose(om, o1, atol=1e-15)
    np.testing.assert_allclose(lm, a, atol=1e-15)
    # all -inf -> (0, -inf)
    om, lm = oracle.merge(np.stack([o1, o2]), np.full((2, r), -np.inf))
    assert np.all(om == 0) and np.all(lm == -np.inf)
    # weights e^a/(e^a+e^b)
    b = a - 1.0
    om, lm = oracle.merge(np.stack([o1, o2]), np.stack([a, b]))
    w1 = 1.0 / (1.0 + np.exp(-1.0))
    np.testing.assert_allclose(om, w1 * o1 + (1 - w1) * o2, atol=1e-14)
    np.testing.assert_allclose(lm, a + np.log1p(np.exp(-1.0)), atol=1e-14)


# --------------------------------------------------------------------------
# Pair counts and tile classes: closed forms, brute force, the pages' examples
# --------------------------------------------------------------------------
def test_pair_counts_closed_forms():
    assert oracle.pair_count(W.causal_s256(False).slices, 256) == 256 * 257 // 2 == 32896
    w2 = W.varlen_causal_t16384(False)
    assert oracle.pair_count(w2.slices, w2.sq) == sum(L * (L + 1) // 2 for L in w2.extra["lengths"])
    w3 = W.block_sparse_strided_s32768(False)
    assert oracle.pair_count(w3.slices, w3.sq) == 4192 * 128 * 128 + 256 * (128 * 129 // 2)
    w5 = W.kv_split_q8192(False)
    assert oracle.pair_count(w5.slices, w5.sq) == 7 * 8192 ** 2 + 8192 * 8193 // 2


def brute_tile_csr(slices, sq, sk, bq, bk):
    m = dense_mask(slices, sq, sk)
    n_qt, n_kt = -(-sq // bq), -(-sk // bk)
    row_ptr, col, tag = [0], [], []
    for qt in range(n_qt):
        for kt in range(n_kt):
            blk = m[qt * bq:(qt + 1) * bq, kt * bk:(kt + 1) * bk]
            c = int(blk.sum())
            if c:
                col.append(kt)
                tag.append(1 if c == blk.size else 2)
        row_ptr.append(len(col))
    return np.array(row_ptr), np.array(col, np.int64), np.array(tag, np.int64)


@pytest.mark.parametrize("bq,bk", [(16, 16), (16, 32), (32, 16), (64, 64), (7, 5)])
def test_tile_csr_brute_force(bq, bk):
    rng = np.random.default_rng(bq * 100 + bk)
    for _ in range(8):
        sq, sk = int(rng.integers(1, 200)), int(rng.integers(1, 200))
        slices = W.random_slices(rng, sq, sk, int(rng.integers(0, 6)))
        rp, col, tag = oracle.tile_csr(slices, sq, sk, bq, bk)
        rp2, col2, tag2 = brute_tile_csr(slices, sq, sk, bq, bk)
        assert np.array_equal(rp, rp2) and np.array_equal(col, col2) and np.array_equal(tag, tag2)


def test_tile_counts_closed_forms():
    _, _, tag = oracle.tile_csr(W.causal_s256(False).slices, 256, 256, 128, 128)
    assert (tag == 1).sum() == 1 and (tag == 2).sum() == 2
    w3 = W.block_sparse_strided_s32768(False)
    _, _, tag = oracle.tile_csr(w3.slices, w3.sq, w3.sk, 128, 128)
    assert (tag == 1).sum() == 4192 and (tag == 2).sum() == 256
    w5 = W.kv_split_q8192(False)
    diag = w5.extra["chunk_slices"][7]
    _, _, tag = oracle.tile_csr(diag, 8192, 8192, 128, 128)
    assert (tag == 1).sum() == 2016 and (tag == 2).sum() == 64


def test_pages_causal_grid_totals():
    """UltraAttn 4.1: a causal P x P grid is P(P-1)/2 Full + P Causal blocks; with the
    page's weights (1, 0.5) the totals are the printed 2, 4.5, 8, 12.5."""
    g = json.load(open(os.path.join(GOLDEN, "ultraattn_causal_grid.json")))
    wf, wc = g["weights"]["full"], g["weights"]["causal"]
    for row in g["rows"]:
        p, blk = row["P"], 16
        s = p * blk
        _, _, tag = oracle.tile_csr([(0, s, 0, s, W.CAUSAL)], s, s, blk, blk)
        total = wf * (tag == 1).sum() + wc * (tag == 2).sum()
        assert total == row["total"]
        assert total / g["n_gpus"] == row["avg"]


def test_pages_ring_example_active_blocks():
    """UltraAttn 1: first block column plus block diagonal on a 4 x 4 grid = 7 blocks."""
    g = json.load(open(os.path.join(GOLDEN, "ultraattn_ring_example.json")))
    n, blk = g["grid"], 8
    codes = np.zeros((n, n), np.uint8)
    codes[:, 0] = 1
    codes[np.arange(n), np.arange(n)] = 1
    slices = W.block_slices(codes, blk, blk, n * blk, n * blk)
    _, col, _ = oracle.tile_csr(slices, n * blk, n * blk, blk, blk)
    assert len(col) == g["active_blocks"]
