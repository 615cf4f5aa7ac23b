"""Device mask compiler (bsfa_dcsr_build) against the host compiler and the CSR oracle:
row_ptr, col, tag, piece_ptr and pieces equal entry for entry, the totals equal the
plan's, and row_ptr / col / tag equal the oracle's tile classification."""
import numpy as np
import pytest

import oracle
from block_sparse_flash_csr_amd import api
from block_sparse_flash_csr_amd import workloads as W

from gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    api.library()
    yield
    torch.cuda.synchronize()


def check(slices, sq, sk, bq, bk, what, with_oracle=True):
    plan = api.Plan.from_slices(slices, sq, sk, 1, 1, 64, bq=bq, bk=bk)
    dc = api.DeviceCsr(slices, sq, sk, bq=bq, bk=bk)
    v = dc.view()
    rp, col, tag, pp, pcs = dc.export()
    hrp, hcol, htag = plan.csr()
    hpp, hpcs = plan.pieces()
    inf = plan.info()
    assert np.array_equal(rp, hrp), f"{what}: row_ptr"
    assert np.array_equal(col, hcol), f"{what}: col"
    assert np.array_equal(tag, htag), f"{what}: tag"
    assert np.array_equal(pp, hpp), f"{what}: piece_ptr"
    assert np.array_equal(pcs, hpcs), f"{what}: pieces"
    for k in ("nnz", "n_full", "n_partial", "n_pieces", "pairs"):
        assert v[k] == inf[k], f"{what}: {k} {v[k]} != {inf[k]}"
    if with_oracle:
        orp, ocol, otag = oracle.tile_csr(slices, sq, sk, bq, bk)
        assert np.array_equal(rp, orp) and np.array_equal(col, ocol) and np.array_equal(tag, otag), what
    dc.close()
    return v


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_workloads(cfg):
    w = W.CONFIGS[cfg](with_inputs=False)
    v = check(w.slices, w.sq, w.sk, 128, 128, w.name)
    say(f"{w.name}: nnz {v['nnz']} ({v['n_full']} F + {v['n_partial']} P), {v['touches']} touches")


def test_workload5_chunks_and_unsplit():
    w = W.config5(with_inputs=False)
    c = w.extra["chunk"]
    for sl in w.extra["chunk_slices"]:
        check(sl, c, c, 128, 128, "config5 chunk")
    check(w.slices, w.sq, w.sk, 128, 128, "config5 unsplit")


@pytest.mark.parametrize("bq,bk", [(16, 16), (16, 32), (32, 16), (64, 128), (128, 128), (128, 64),
                                   (7, 13), (256, 256), (512, 200)])
def test_random_masks(bq, bk):
    rng = np.random.default_rng(bq * 1000 + bk + 17)
    for _ in range(20):
        sq, sk = int(rng.integers(1, 700)), int(rng.integers(1, 700))
        slices = W.random_slices(rng, sq, sk, int(rng.integers(0, 12)))
        check(slices, sq, sk, bq, bk, f"random bq={bq} bk={bk}")


def test_edge_cases():
    check([], 300, 200, 128, 128, "no slices")
    check([(5, 5, 0, 10, 0), (0, 10, 7, 7, 1)], 300, 200, 128, 128, "empty slices")
    # several partial slices whose union covers a tile: full, no pieces
    check([(0, 128, 0, 64, 0), (0, 128, 64, 128, 0), (0, 64, 128, 256, 0), (64, 128, 128, 256, 0)],
          128, 256, 128, 128, "union-full tiles")
    # overlapping causal + full slices over the same tiles (duplicate incidences)
    check([(0, 512, 0, 512, 1), (0, 512, 0, 512, 1), (100, 400, 50, 300, 0)], 512, 512, 128, 128,
          "duplicates")
    check([(0, 1, 0, 1, 0)], 1, 1, 128, 128, "one pair")


@pytest.mark.parametrize("kind", ["causal", "strided"])
def test_benchmark_sizes_524288(kind):
    """The 524,288-token masks the benchmark times: every array equal to the host plan's
    (the oracle's row-by-row classification would take minutes at this size)."""
    S = 524288
    if kind == "causal":
        sl = [(0, S, 0, S, 1)]
    else:
        sl = W.block_slices(W.strided_block_codes(S // 128, 8), 128, 128, S, S)
    v = check(api.slice_array(sl), S, S, 128, 128, f"{kind} s{S}", with_oracle=False)
    say(f"{kind} s{S}: nnz {v['nnz']} ({v['n_full']} F + {v['n_partial']} P), {v['touches']} touches")
