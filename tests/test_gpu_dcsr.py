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
    w = W.WORKLOADS[cfg](with_inputs=False)
    v = check(w.slices, w.sq, w.sk, 128, 128, w.name)
    say(f"{w.name}: nnz {v['nnz']} ({v['n_full']} F + {v['n_partial']} P), {v['touches']} touches")


def test_workload5_chunks_and_unsplit():
    w = W.kv_split_q8192(with_inputs=False)
    c = w.extra["chunk"]
    for sl in w.extra["chunk_slices"]:
        check(sl, c, c, 128, 128, "kv split q8192 chunk")
    check(w.slices, w.sq, w.sk, 128, 128, "kv split q8192 unsplit")


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


def _same_plan(a, b, what):
    for name in ("csr", "pieces", "schedule", "units"):
        for x, y in zip(getattr(a, name)(), getattr(b, name)()):
            assert np.array_equal(x, y), f"{what}: {name}"
    ia, ib = a.info(), b.info()
    for k in ("nnz", "n_full", "n_partial", "n_pieces", "pairs", "n_items", "n_bins", "n_units", "n_splits"):
        assert ia[k] == ib[k], f"{what}: {k}"


@pytest.mark.parametrize("cfg", [2, 3])
def test_plan_from_device_csr_equals_host_plan(cfg):
    """A plan over the device-compiled CSR is the host plan: CSR, pieces, schedule and
    units equal, and the forward and backward outputs bit-identical."""
    import torch
    w = W.WORKLOADS[cfg]()
    say(f"plan from device CSR: {w.name}")
    host = api.Plan.from_slices(w.slices, w.sq, w.sk, w.hq, w.hkv, w.d)
    dc = api.DeviceCsr(w.slices, w.sq, w.sk)
    dev = dc.plan(w.hq, w.hkv, w.d)
    dc.close()                      # the plan owns copies of everything it needs
    _same_plan(host, dev, w.name)
    q, k, v = api.to_device_bf16(w.q), api.to_device_bf16(w.k), api.to_device_bf16(w.v)
    host.upload()
    dev.upload()
    oh, lh = api.attn_fwd(q, k, v, host, w.scale)
    od, ld = api.attn_fwd(q, k, v, dev, w.scale)
    g = api.to_device_bf16(W.random_grad(np.random.default_rng(cfg), w.sq, w.hq, w.d))
    gh = api.attn_bwd(q, k, v, g, lh, host, w.scale)
    gd = api.attn_bwd(q, k, v, g, ld, dev, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(oh.view(torch.int16), od.view(torch.int16)) and torch.equal(lh, ld)
    for x, y in zip(gh, gd):
        assert torch.equal(x, y)
    host.close()
    dev.close()


def test_plan_from_device_csr_at_65536_tokens():
    """A causal mask of 65,536 tokens (131,328 entries: the column view's stable sort runs
    over 33 workgroups of keys in two digit passes, the compiler's key sort over three):
    the plan over the device CSR equals the host plan, and the forward and the backward,
    which walks the column view, are bit-identical."""
    import torch
    S, hq, hkv, d = 65536, 2, 1, 64
    sl = [(0, S, 0, S, 1)]
    say(f"plan from device CSR: causal s{S} hq={hq} hkv={hkv} d={d}")
    host = api.Plan.from_slices(sl, S, S, hq, hkv, d)
    dc = api.DeviceCsr(sl, S, S)
    dev = dc.plan(hq, hkv, d)
    dc.close()
    assert host.info()["nnz"] == 512 * 513 // 2
    _same_plan(host, dev, f"causal s{S}")
    rng = np.random.default_rng(65536)
    qb, kb, vb = W.random_inputs(rng, S, S, hq, hkv, d)
    q, k, v = api.to_device_bf16(qb), api.to_device_bf16(kb), api.to_device_bf16(vb)
    host.upload()
    dev.upload()
    oh, lh = api.attn_fwd(q, k, v, host, 0.125)
    od, ld = api.attn_fwd(q, k, v, dev, 0.125)
    g = api.to_device_bf16(W.random_grad(rng, S, hq, d))
    gh = api.attn_bwd(q, k, v, g, lh, host, 0.125)
    gd = api.attn_bwd(q, k, v, g, ld, dev, 0.125)
    torch.cuda.synchronize()
    assert torch.equal(oh.view(torch.int16), od.view(torch.int16)) and torch.equal(lh, ld)
    for name, x, y in zip(("dQ", "dK", "dV"), gh, gd):
        assert torch.equal(x, y), name
    host.close()
    dev.close()


def test_plan_from_device_csr_split_rows_and_ragged_tails():
    """Few query rows against long keys (rows split into parts), ragged extents, head
    dim 64 and 64-key plan tiles; the forward on the device CSR's plan equals the host
    plan's bit for bit."""
    import torch
    rng = np.random.default_rng(31)
    for sq, sk, hq, hkv, d, bk in ((100, 9000, 8, 2, 128, 128), (333, 1001, 4, 4, 64, 128),
                                   (517, 700, 6, 2, 128, 64)):
        say(f"plan from device CSR: sq={sq} sk={sk} hq={hq} hkv={hkv} d={d} bk={bk}")
        slices = W.random_slices(rng, sq, sk, 6) + [(0, sq, 0, sk, 1)]
        host = api.Plan.from_slices(slices, sq, sk, hq, hkv, d, bk=bk)
        dc = api.DeviceCsr(slices, sq, sk, bk=bk)
        with pytest.raises(api.BsfaError):
            dc.plan(hq + 1, hkv + 1, d) if (hq + 1) % (hkv + 1) else dc.plan(hq, hkv + 1, d)
        dev = dc.plan(hq, hkv, d)
        dc.close()
        _same_plan(host, dev, f"sq={sq} sk={sk}")
        qb, kb, vb = W.random_inputs(rng, sq, sk, hq, hkv, d)
        q, k, v = api.to_device_bf16(qb), api.to_device_bf16(kb), api.to_device_bf16(vb)
        oh, lh = api.attn_fwd(q, k, v, host.upload(), 0.1)
        od, ld = api.attn_fwd(q, k, v, dev.upload(), 0.1)
        torch.cuda.synchronize()
        assert torch.equal(oh.view(torch.int16), od.view(torch.int16))
        assert torch.equal(lh.nan_to_num(neginf=-1e30), ld.nan_to_num(neginf=-1e30))
        host.close()
        dev.close()


def test_plan_from_device_csr_of_an_empty_mask():
    """No slice at all: the plan has no tiles, every row gets O = 0 and LSE = -inf."""
    import torch
    sq, sk, hq, hkv, d = 300, 200, 2, 1, 128
    dc = api.DeviceCsr([], sq, sk)
    dev = dc.plan(hq, hkv, d)
    dc.close()
    host = api.Plan.from_slices([], sq, sk, hq, hkv, d)
    _same_plan(host, dev, "empty mask")
    assert dev.info()["nnz"] == 0
    rng = np.random.default_rng(5)
    qb, kb, vb = W.random_inputs(rng, sq, sk, hq, hkv, d)
    o, lse = api.attn_fwd(api.to_device_bf16(qb), api.to_device_bf16(kb), api.to_device_bf16(vb),
                          dev.upload(), 0.1)
    torch.cuda.synchronize()
    assert bool((o.float() == 0).all()) and bool(torch.isneginf(lse).all())
    host.close()
    dev.close()


def test_device_compiles_from_several_host_threads():
    """Four host threads compile masks on the GPU at once (each on its own stream; the
    pinned staging images are shared) and upload plans in between; every CSR equals the
    host compiler's."""
    import threading
    import torch
    rng = np.random.default_rng(59)
    cases = []
    for _ in range(6):
        sq, sk = int(rng.integers(100, 900)), int(rng.integers(100, 900))
        cases.append((W.random_slices(rng, sq, sk, int(rng.integers(1, 12))), sq, sk))
    refs = []
    for sl, sq, sk in cases:
        p = api.Plan.from_slices(sl, sq, sk, 1, 1, 64)
        refs.append(p.csr())
        p.close()
    streams = [torch.cuda.Stream() for _ in range(4)]
    errors = []

    def worker(t):
        try:
            torch.cuda.set_device(0)
            for i in range(12):
                c = (t + i) % len(cases)
                sl, sq, sk = cases[c]
                dc = api.DeviceCsr(sl, sq, sk, stream=streams[t])
                up = api.Plan.from_slices(sl, sq, sk, 2, 1, 128).upload(streams[t])   # shares the images
                rp, col, tag, _, _ = dc.export()
                dc.close()
                up.close()
                if not (np.array_equal(rp, refs[c][0]) and np.array_equal(col, refs[c][1])
                        and np.array_equal(tag, refs[c][2])):
                    errors.append(f"thread {t} iteration {i}: CSR of case {c} differs")
        except Exception as e:   # reported below, in the test's own thread
            errors.append(repr(e))

    say("device compiles from 4 host threads x 12")
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors


def check_blocks(codes, sq, sk, bq, bk, what):
    """bsfa_dcsr_build_blocks against the host plan of the same block map (blocks = tiles)."""
    plan = api.Plan.from_blocks(codes, bq, bk, sq, sk, 1, 1, 64, bq=bq, bk=bk)
    dc = api.DeviceCsr.from_blocks(codes, sq, sk, bq=bq, bk=bk)
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
    assert v["touches"] == v["nnz"]
    dc.close()
    plan.close()
    return v


@pytest.mark.parametrize("bq,bk", [(128, 128), (64, 128), (128, 64), (128, 256), (16, 48), (1, 7)])
def test_block_codes_compiled_on_the_device(bq, bk):
    """Random code maps (densities 0 to 1, every code), maps shorter, exactly as long and
    longer than the tile grid, ragged last rows and columns, single-row blocks."""
    rng = np.random.default_rng(bq * 7919 + bk)
    for t in range(24):
        sq, sk = int(rng.integers(1, 1200)), int(rng.integers(1, 1200))
        nqt, nkt = -(-sq // bq), -(-sk // bk)
        nbq = max(0, nqt + int(rng.integers(-2, 3)))
        nbk = max(0, nkt + int(rng.integers(-2, 3)))
        dens = float(rng.uniform(0, 1))
        codes = np.where(rng.random((nbq, nbk)) < dens, rng.integers(1, 3, (nbq, nbk)), 0).astype(np.uint8)
        check_blocks(codes, sq, sk, bq, bk, f"blocks bq={bq} bk={bk} sq={sq} sk={sk} map {nbq}x{nbk}")


def test_block_codes_edge_cases():
    check_blocks(np.zeros((0, 0), np.uint8), 300, 200, 128, 128, "empty map")
    check_blocks(np.zeros((3, 2), np.uint8), 300, 200, 128, 128, "all-empty map")
    check_blocks(np.full((1, 1), 2, np.uint8), 1, 1, 128, 128, "one causal pair")
    check_blocks(np.full((4, 4), 2, np.uint8), 385, 390, 128, 128, "causal, ragged last row of one token")
    check_blocks(np.full((2, 2), 1, np.uint8), 0, 0, 128, 128, "no rows, no keys")


def test_block_codes_refuse_a_code_above_2():
    codes = np.zeros((3, 3), np.uint8)
    codes[2, 1] = 3
    with pytest.raises(api.BsfaError) as e:
        api.DeviceCsr.from_blocks(codes, 384, 384)
    assert e.value.status == 5


def test_strided_blocks_device_plan_and_forward():
    """The strided workload's code map compiled on the device: its plan equals the host
    plan built from the same map, and the forward over it is bit-identical."""
    import torch
    w = W.block_sparse_strided_s32768()
    codes = W.strided_block_codes(w.sq // 128, 8)
    check_blocks(codes, w.sq, w.sk, 128, 128, "strided s32768")
    hp = api.Plan.from_blocks(codes, 128, 128, w.sq, w.sk, w.hq, w.hkv, w.d).upload()
    dc = api.DeviceCsr.from_blocks(codes, w.sq, w.sk)
    dp = dc.plan(w.hq, w.hkv, w.d)
    dc.close()
    _same_plan(dp, hp, "strided s32768 from blocks")
    q, k, v = api.to_device_bf16(w.q), api.to_device_bf16(w.k), api.to_device_bf16(w.v)
    o1, l1 = api.attn_fwd(q, k, v, hp, w.scale)
    o2, l2 = api.attn_fwd(q, k, v, dp.upload(), w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    say("strided s32768: device plan from the block map equals the host plan; forward bit-identical")
    hp.close()
    dp.close()


def test_block_codes_524288():
    """The benchmark's strided map at 524,288 tokens (4096 x 4096 blocks)."""
    S = 524288
    v = check_blocks(W.strided_block_codes(S // 128, 8), S, S, 128, 128, "strided blocks s524288")
    say(f"strided blocks s{S}: nnz {v['nnz']} ({v['n_full']} F + {v['n_partial']} P)")
