"""Pins of the fp64 backward oracle against things other than its own formulas:
central finite differences of the (separately pinned) fp64 forward, closed forms of
one-key rows and of identical keys, and its bf16 entry against its fp64 entry."""
import numpy as np
import pytest

import oracle
from block_sparse_flash_csr_amd import workloads as W


def _loss(q, k, v, g, slices, scale):
    o, _ = oracle.attn_fwd_f64(q, k, v, slices, scale)
    return float(np.sum(o * g))


@pytest.mark.parametrize("seed,sq,sk,hq,hkv,d", [(0, 6, 9, 2, 1, 4), (1, 5, 5, 1, 1, 3),
                                                  (2, 7, 4, 4, 2, 2)])
def test_gradients_match_central_differences(seed, sq, sk, hq, hkv, d):
    rng = np.random.default_rng(seed)
    # random slices (causal and full, overlapping) plus one row left without keys
    slices = [s for s in W.random_slices(rng, sq, sk, 4) if not (s[0] <= sq - 1 < s[1])]
    slices.append((0, max(1, sq - 2), 0, sk, 1))
    q = rng.standard_normal((sq, hq, d))
    k = rng.standard_normal((sk, hkv, d))
    v = rng.standard_normal((sk, hkv, d))
    g = rng.standard_normal((sq, hq, d))
    scale = 0.7
    dq, dk, dv = oracle.attn_bwd_f64(q, k, v, g, slices, scale)
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], g, slices, scale) -
                       _loss(args_m["q"], args_m["k"], args_m["v"], g, slices, scale)) / (2 * eps)
        assert np.max(np.abs(fd - grad)) < 1e-7 * max(1.0, np.max(np.abs(grad))), name
    # the row without keys gets no gradient
    assert np.all(dq[sq - 1] == 0.0)


def test_one_key_rows():
    """A row that admits one key has P = 1 and D = dO . v_j = dP: dS = 0, so dQ = dK = 0
    and dV_j is the plain sum of the dO rows that attend to j."""
    rng = np.random.default_rng(3)
    sq, sk, d = 8, 5, 6
    keys = [int(j) for j in rng.integers(0, sk, size=sq)]
    slices = [(i, i + 1, keys[i], keys[i] + 1, 0) for i in range(sq)]
    q = rng.standard_normal((sq, 1, d))
    k = rng.standard_normal((sk, 1, d))
    v = rng.standard_normal((sk, 1, d))
    g = rng.standard_normal((sq, 1, d))
    dq, dk, dv = oracle.attn_bwd_f64(q, k, v, g, slices, 0.5)
    assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12
    want = np.zeros((sk, 1, d))
    for i, j in enumerate(keys):
        want[j, 0] += g[i, 0]
    assert np.max(np.abs(dv - want)) < 1e-12


def test_identical_keys_give_no_query_gradient():
    """The dS of a row sums to zero (sum_j P (dP - D) = D - D), so with every key equal
    dQ_i = scale * k * sum_j dS_ij = 0."""
    rng = np.random.default_rng(4)
    sq, sk, d = 6, 7, 5
    q = rng.standard_normal((sq, 2, d))
    k = np.repeat(rng.standard_normal((1, 1, d)), sk, axis=0)
    v = rng.standard_normal((sk, 1, d))
    g = rng.standard_normal((sq, 2, d))
    dq, _, _ = oracle.attn_bwd_f64(q, k, v, g, [(0, sq, 0, sk, 1), (2, 5, 0, 3, 0)], 0.9)
    assert np.max(np.abs(dq)) < 1e-12


def test_bf16_entry_equals_f64_entry():
    rng = np.random.default_rng(5)
    sq, sk, hq, hkv, d = 9, 11, 2, 2, 8
    qb, kb, vb = W.random_inputs(rng, sq, sk, hq, hkv, d)
    gb = W.bf16_bits(rng.standard_normal((sq, hq, d), dtype=np.float32))
    slices = W.random_slices(rng, sq, sk, 3)
    a = oracle.attn_bwd(qb, kb, vb, gb, slices, 0.3, n_threads=2)
    f = [W.bf16_to_f32(x).astype(np.float64) for x in (qb, kb, vb, gb)]
    b = oracle.attn_bwd_f64(*f, slices, 0.3)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("seed,sq,sk,hq,hkv,d,n", [(41, 37, 29, 4, 2, 16, 4), (42, 50, 50, 3, 1, 8, 3)])
def test_sampled_backward_equals_full_pass(seed, sq, sk, hq, hkv, d, n):
    """The sampled gradients add the same terms in the same order as the full pass,
    so they agree with it exactly (rows without keys and unreached keys included)."""
    rng = np.random.default_rng(seed)
    slices = W.random_slices(rng, sq, sk, n) + [(5, 9, 0, 0, 0)]
    qb, kb, vb = W.random_inputs(rng, sq, sk, hq, hkv, d)
    gb = W.random_grad(rng, sq, hq, d)
    dq, dk, dv = oracle.attn_bwd(qb, kb, vb, gb, slices, 0.3)
    rows = [(h, i) for h in range(hq) for i in range(sq)]
    keys = [(g, j) for g in range(hkv) for j in range(sk)]
    sq_, sk_, sv_ = oracle.attn_bwd_sampled(qb, kb, vb, gb, slices, 0.3, rows=rows, keys=keys)
    assert np.array_equal(sq_, np.stack([dq[i, h] for h, i in rows]))
    assert np.array_equal(sk_, np.stack([dk[j, g] for g, j in keys]))
    assert np.array_equal(sv_, np.stack([dv[j, g] for g, j in keys]))
