"""Pins of the oracle's route-and-align step (CPU only): a hand-worked golden,
a sort-based brute force and the structural invariants."""
import json
import os

import numpy as np
import pytest

import workloads as W
from oracle import moe as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute(topk_ids, start, n_local, B):
    """Independent construction: a stable argsort of the local ids with the
    off-slice slots removed, then each expert run padded to a multiple of B."""
    ids = np.asarray(topk_ids).reshape(-1)
    local = np.array([i - start if start <= i < start + n_local else -1 for i in ids])
    order = np.argsort(local, kind="stable")
    order = [int(o) for o in order if local[o] >= 0]
    numel = ids.size
    out, blocks = [], []
    i = 0
    while i < len(order):
        e = local[order[i]]
        j = i
        while j < len(order) and local[order[j]] == e:
            j += 1
        run = order[i:j]
        pad = (-len(run)) % B
        out += run + [numel] * pad
        blocks += [int(e)] * ((len(run) + pad) // B)
        i = j
    return out, blocks


def test_golden_small():
    g = json.load(open(os.path.join(GOLDEN, "align_small.json")))
    s, e, n, loc = O.moe_align(np.array(g["topk_ids"], dtype=np.int32), g["expert_start"],
                               g["n_local"], g["block_m"])
    assert s.tolist() == g["sorted_token_ids"]
    assert e.tolist() == g["expert_ids"]
    assert n == g["num_tokens_post_padded"]
    assert loc.tolist() == g["slot_local_ids"]


@pytest.mark.parametrize("M,k,E_glob,start,n_local,B", [
    (1, 8, 256, 0, 32, 16), (7, 2, 8, 0, 8, 16), (123, 2, 8, 0, 8, 64), (64, 8, 256, 32, 32, 8),
    (333, 4, 128, 0, 128, 48), (50, 3, 10, 7, 3, 1), (4, 8, 256, 200, 56, 32),
])
def test_matches_sort_brute_force(M, k, E_glob, start, n_local, B):
    rng = np.random.default_rng([M, k, B])
    ids = np.argsort(rng.random((M, E_glob)), axis=1)[:, :k].astype(np.int32)
    s, e, n, loc = O.moe_align(ids, start, n_local, B)
    ref_s, ref_b = _brute(ids, start, n_local, B)
    assert n == len(ref_s)
    assert s[:n].tolist() == ref_s
    assert e[:len(ref_b)].tolist() == ref_b
    assert np.all(s[n:] == M * k) and np.all(e[len(ref_b):] == -1)


def _check_invariants(ids, start, n_local, B):
    s, e, n, loc = O.moe_align(ids, start, n_local, B)
    numel = ids.size
    cap, cap_b = O.align_capacity(numel, n_local, B)
    assert s.size == cap and e.size == cap_b and cap == cap_b * B
    assert n % B == 0 and n <= cap
    live = s[:n][s[:n] < numel]
    flat_local = loc.reshape(-1)
    # every live slot appears exactly once, dead slots never
    assert sorted(live.tolist()) == [i for i in range(numel) if flat_local[i] >= 0]
    # blocks: expert ids non-decreasing over [0, n/B), each entry routes there
    be = e[: n // B]
    assert np.all(np.diff(be) > -1) and np.all(be >= 0)
    for b in range(n // B):
        blk = s[b * B:(b + 1) * B]
        real = blk[blk < numel]
        assert real.size > 0 and np.all(flat_local[real] == be[b])
        assert np.all(np.diff(real) > 0)   # ascending inside a block
    # segment lengths are ceil(count / B) * B
    for x in range(n_local):
        cnt = int(np.sum(flat_local == x))
        assert int(np.sum(be == x)) * B == -(-cnt // B) * B


@pytest.mark.parametrize("name", [W.INT4_SMALL, W.NVFP4_DECODE, W.NVFP4_ZIPF, W.MXFP4_SWIGLU])
def test_invariants_on_workload_routing(name):
    wl = W.WORKLOADS[name]
    M = min(wl.Ms[-1], 512)
    inp = W.make_inputs(wl, M)
    B = 16
    _check_invariants(inp.topk_ids, wl.expert_start, wl.n_local, B)


def test_capacity_is_tight():
    # every expert gets count = 1 (mod B): the padded total reaches the bound
    B, n_local = 8, 5
    ids = np.array([[e] for e in range(n_local)] * 9, dtype=np.int32)  # 9 per expert
    numel = ids.size
    s, e, n, _ = O.moe_align(ids, 0, n_local, B)
    assert n == numel + n_local * (B - 1)
    assert O.align_capacity(numel, n_local, B)[0] >= n


def test_all_off_slice_and_empty():
    ids = np.full((5, 4), 99, dtype=np.int32)
    s, e, n, loc = O.moe_align(ids, 0, 32, 16)
    assert n == 0 and np.all(s == 20) and np.all(e == -1) and np.all(loc == -1)
    s, e, n, loc = O.moe_align(np.zeros((0, 8), dtype=np.int32), 0, 32, 16)
    assert n == 0 and s.size == 0 and e.size == 0


def test_route_local_brute_force():
    rng = np.random.default_rng(5)
    ids = rng.integers(0, 256, size=(64, 8)).astype(np.int32)
    got = O.route_local(ids, 96, 32)
    for (t, s), v in np.ndenumerate(ids):
        assert got[t, s] == (v - 96 if 96 <= v < 128 else -1)
