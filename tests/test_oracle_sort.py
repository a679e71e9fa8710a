"""Pins of the oracle's routing plan: a hand-derived worked example
(tests/golden), an independent brute force (stable sort of (expert, route))
and the plan invariants on every workload's routing."""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from plan_checks import brute_force_plan, capacity, check_invariants


def _cmp(plan, ref):
    assert np.array_equal(plan.expanded_to_permuted, ref["expanded_to_permuted"])
    assert np.array_equal(plan.permuted_to_expanded, ref["permuted_to_expanded"])
    assert np.array_equal(plan.tile_to_expert, ref["tile_to_expert"])
    assert np.array_equal(plan.tile_to_mn_limit, ref["tile_to_mn_limit"])
    assert plan.num_tiles == ref["num_tiles"]
    assert np.array_equal(plan.expert_offsets, ref["expert_offsets"])
    assert np.array_equal(plan.expert_counts, ref["expert_counts"])


def test_worked_example(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "sort_worked_example.json")))
    ids = np.array(ex["topk_ids"], np.int32)
    assert oracle.route_slots(ids.shape[0], ids.shape[1], ex["num_local_experts"], ex["tile"]) == ex["route_slots"]
    plan = oracle.sort(ids, ex["num_local_experts"], ex["local_expert_offset"], ex["tile"])
    _cmp(plan, ex)


CASES = [
    # (M, k, E_g, E_l, offset, T, seed)
    (1, 1, 1, 1, 0, 1, 0), (3, 2, 4, 4, 0, 2, 1), (17, 4, 16, 5, 3, 8, 2), (64, 8, 256, 32, 0, 16, 3),
    (100, 6, 64, 64, 0, 32, 4), (33, 3, 10, 3, 7, 4, 5), (200, 2, 8, 1, 5, 128, 6), (50, 8, 256, 32, 224, 64, 7),
]


@pytest.mark.parametrize("case", CASES)
def test_matches_brute_force(case):
    M, k, Eg, El, off, T, seed = case
    rng = np.random.default_rng(seed)
    ids = rng.integers(-2, Eg + 2, (M, k)).astype(np.int32)   # includes out-of-range ids
    plan = oracle.sort(ids, El, off, T)
    _cmp(plan, brute_force_plan(ids, El, off, T))
    check_invariants(ids, El, off, T, plan.expanded_to_permuted, plan.permuted_to_expanded, plan.tile_to_expert,
                     plan.tile_to_mn_limit, plan.num_tiles, plan.expert_offsets, plan.expert_counts)


def test_edge_cases():
    # all routes non-local
    ids = np.full((5, 3), 9, np.int32)
    plan = oracle.sort(ids, 4, 0, 8)
    assert plan.num_tiles == 0 and np.all(plan.expanded_to_permuted == -1) and np.all(plan.permuted_to_expanded == -1)
    # every route to one expert, duplicates inside a token
    ids = np.zeros((9, 4), np.int32)
    plan = oracle.sort(ids, 2, 0, 16)
    _cmp(plan, brute_force_plan(ids, 2, 0, 16))
    assert plan.expert_counts[0] == 36 and plan.num_tiles == 3
    # no tokens
    ids = np.zeros((0, 8), np.int32)
    plan = oracle.sort(ids, 32, 0, 64)
    assert plan.num_tiles == 0 and plan.permuted_to_expanded.size == 0


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_routing_invariants(name):
    wl = synth.WORKLOADS[name]
    ids, w = synth.make_routing(wl)
    for T in (16, 64, 256):
        plan = oracle.sort(ids, wl.num_local_experts, wl.local_expert_offset, T)
        check_invariants(ids, wl.num_local_experts, wl.local_expert_offset, T, plan.expanded_to_permuted,
                         plan.permuted_to_expanded, plan.tile_to_expert, plan.tile_to_mn_limit, plan.num_tiles,
                         plan.expert_offsets, plan.expert_counts)
        assert plan.permuted_to_expanded.size == capacity(wl.M, wl.top_k, wl.num_local_experts, T)
