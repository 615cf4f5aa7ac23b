"""Min-heap greedy scheduler: coverage, conservation, Graham's LPT bound against brute-force
optima, determinism, and the pages' block weights / imbalance table."""
import itertools
import json
import os

import numpy as np
import pytest

from block_sparse_flash_csr_amd import api
from block_sparse_flash_csr_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_opt(costs, m):
    best = float("inf")
    for assign in itertools.product(range(m), repeat=len(costs)):
        loads = [0.0] * m
        for c, b in zip(costs, assign):
            loads[b] += c
        best = min(best, max(loads))
    return best


def test_lpt_bound_against_brute_force():
    rng = np.random.default_rng(0)
    for trial in range(60):
        n = int(rng.integers(1, 9))
        m = int(rng.integers(1, 4))
        costs = np.round(rng.uniform(0.5, 10, size=n), 2).astype(np.float32)
        bin_of, load, mk = api.lpt_assign(costs, m)
        opt = brute_opt([float(c) for c in costs], m)
        assert mk <= (4.0 / 3.0 - 1.0 / (3 * m)) * opt + 1e-5
        assert abs(load.sum() - costs.astype(np.float64).sum()) < 1e-4
        for b in range(m):
            assert abs(load[b] - costs[bin_of == b].astype(np.float64).sum()) < 1e-4


def test_lpt_is_deterministic_and_follows_the_greedy_rule():
    costs = np.array([3, 3, 2, 2, 2, 1], np.float32)
    bin_of, load, mk = api.lpt_assign(costs, 2)
    # 3->b0, 3->b1, 2->b0, 2->b1, 2->b0 (tie 5,5 -> b0), 1->b1
    assert list(bin_of) == [0, 1, 0, 1, 0, 1]
    assert mk == 7.0
    for _ in range(3):
        b2, _, _ = api.lpt_assign(costs, 2)
        assert np.array_equal(b2, bin_of)


def _check_plan_schedule(plan):
    inf = plan.info()
    bin_ptr, items, cost = plan.schedule()
    assert bin_ptr[0] == 0 and bin_ptr[-1] == inf["n_units"]
    assert np.all(np.diff(bin_ptr) >= 0)
    assert sorted(items.tolist()) == list(range(inf["n_units"]))
    loads = np.array([cost[items[bin_ptr[b]:bin_ptr[b + 1]]].astype(np.float64).sum()
                      for b in range(inf["n_bins"])])
    assert abs(loads.sum() - inf["total_cost"]) < 1e-3 * max(1.0, inf["total_cost"])
    assert abs(loads.max() - inf["makespan"]) < 1e-3 * max(1.0, inf["makespan"])
    avg = inf["total_cost"] / inf["n_bins"]
    assert inf["makespan"] <= avg + cost.max() + 1e-3
    return inf, loads


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workload_schedules(cfg):
    w = W.WORKLOADS[cfg](with_inputs=False)
    plan = api.plan_from_workload(w, upload=False)
    inf, loads = _check_plan_schedule(plan)
    assert inf["n_splits"] == 0 and inf["n_units"] == inf["n_items"]   # no row needs splitting
    assert inf["n_bins"] == min(inf["n_items"], 512)
    # repeat build: identical schedule
    plan2 = api.plan_from_workload(w, upload=False)
    for a, b in zip(plan.schedule(), plan2.schedule()):
        assert np.array_equal(a, b)


def test_item_cost_model():
    """Cost of an item = per-item constant + full steps + 1.15 x partial steps (64-key steps)."""
    plan = api.Plan.from_slices([(0, 256, 0, 256, 1)], 256, 256, 1, 1, 128)
    _, _, cost = plan.schedule()
    # q-tile 0: one partial 128-key tile = 2 steps; q-tile 1: one full + one partial tile
    assert abs(cost[0] - (1.0 + 2 * 1.15)) < 1e-5
    assert abs(cost[1] - (1.0 + 2 + 2 * 1.15)) < 1e-5


def test_pages_block_weights_and_imbalance_table():
    """UltraAttn 4.1: full 1, causal 0.5, empty 0; ceil(avg)/avg - 1 for the causal grid."""
    g = json.load(open(os.path.join(GOLDEN, "ultraattn_causal_grid.json")))
    lib = api.library()
    assert lib.bsfa_tile_cost(api.TILE_FULL, g["weights"]["causal"]) == g["weights"]["full"]
    assert lib.bsfa_tile_cost(0, 0.5) == g["weights"]["empty"]
    for row in g["rows"]:
        p, blk = row["P"], 32
        s = p * blk
        plan = api.Plan.from_slices([(0, s, 0, s, 1)], s, s, 1, 1, 64, bq=blk, bk=blk)
        _, _, tag = plan.csr()
        total = sum(lib.bsfa_tile_cost(int(t), g["weights"]["causal"]) for t in tag)
        assert total == row["total"]
        assert total / g["n_gpus"] == row["avg"]
        assert int(np.ceil(total / g["n_gpus"])) == row["max"]
        assert round(lib.bsfa_imbalance_bound(total, g["n_gpus"]), 2) == row["imbalance"]


# ---------------------------------------------------------------------------
# in-call KV split: rows costlier than the per-bin target are cut into parts
# ---------------------------------------------------------------------------
def _check_units(plan):
    inf = plan.info()
    row_ptr, col, tag = plan.csr()
    units = plan.units()
    n_qt, hq = inf["n_qtiles"], inf["hq"]
    assert units.shape == (inf["n_units"], 4)
    # per item, the parts tile the CSR row in order, each part non-empty
    by_item = {}
    for u, (item, eb, ee, slot) in enumerate(units):
        by_item.setdefault(int(item), []).append((int(eb), int(ee), int(slot)))
    assert sorted(by_item) == list(range(hq * n_qt))
    slots = []
    for item, parts in by_item.items():
        qt = item % n_qt
        assert parts[0][0] == row_ptr[qt] and parts[-1][1] == row_ptr[qt + 1]
        for (a0, a1, _), (b0, _, _) in zip(parts, parts[1:]):
            assert a1 == b0
        if len(parts) == 1:
            assert parts[0][2] == -1
        else:
            assert all(p[0] < p[1] for p in parts)
            assert len(parts) <= 16
            first = parts[0][2]
            assert [p[2] for p in parts] == list(range(first, first + len(parts)))
            slots += [p[2] for p in parts]
    assert sorted(slots) == list(range(len(slots)))
    assert inf["n_splits"] == sum(1 for p in by_item.values() if len(p) > 1)
    assert inf["workspace_bytes"] == len(slots) * 128 * (inf["d"] + 1) * 4
    return units


@pytest.mark.parametrize("sq,sk,hq,causal", [(256, 16384, 2, False), (200, 20000, 1, True),
                                              (1024, 65536, 8, False)])
def test_long_rows_are_split_into_balanced_parts(sq, sk, hq, causal):
    slices = [(0, sq, 0, sk, 1 if causal else 0)]
    plan = api.Plan.from_slices(slices, sq, sk, hq, hq, 128)
    inf, loads = _check_plan_schedule(plan)
    units = _check_units(plan)
    assert inf["n_splits"] > 0
    # parts of one row cost about the same (within one entry of 2 steps plus rounding)
    _, _, cost = plan.schedule()
    for item in set(units[:, 0].tolist()):
        c = cost[units[:, 0] == item]
        if len(c) > 1:
            assert c.max() - c.min() <= 2 * 1.15 + 1e-4
    # the split leaves the makespan close to the mean load
    assert inf["makespan"] <= inf["total_cost"] / inf["n_bins"] + cost.max() + 1e-3


def test_short_rows_are_not_split():
    # every row is below the 16-step floor: no split however few the items
    plan = api.Plan.from_slices([(0, 256, 0, 256, 1)], 256, 256, 1, 1, 128)
    inf = plan.info()
    assert inf["n_splits"] == 0 and inf["workspace_bytes"] == 0
    _check_units(plan)
