"""GPU align vs the oracle: bit-exact on every output entry (the whole capacity)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe as O
import quantized_mixture_experts_align_amd as P

pytestmark = pytest.mark.gpu


def _run(ids: np.ndarray, start: int, n_local: int, B: int, slot_ids=True):
    t = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
    s, e, n, loc = P.moe_align(t, start, n_local, B, slot_local_ids=slot_ids)
    torch.cuda.synchronize()
    return (s.cpu().numpy(), e.cpu().numpy(), int(n.cpu().item()),
            None if loc is None else loc.cpu().numpy())


def _check(ids, start, n_local, B):
    print(f"align M={ids.shape[0]} k={ids.shape[1]} start={start} n_local={n_local} B={B}", flush=True)
    gs, ge, gn, gl = _run(ids, start, n_local, B)
    rs, re_, rn, rl = O.moe_align(ids, start, n_local, B)
    assert gn == rn
    assert np.array_equal(gs, rs)
    assert np.array_equal(ge, re_)
    assert np.array_equal(gl, rl)


@pytest.mark.parametrize("name,M,B", [(W.INT4_SMALL, 123, 32), (W.INT4_BIAS, 2304, 128),
                                      (W.NVFP4_DECODE, 1, 16), (W.NVFP4_DECODE, 4, 16), (W.NVFP4_DECODE, 16, 16),
                                      (W.NVFP4_DECODE, 64, 16), (W.NVFP4_ZIPF, 256, 64), (W.NVFP4_ZIPF, 1024, 128),
                                      (W.NVFP4_ZIPF, 4096, 128), (W.MXFP4_SWIGLU, 1, 16), (W.MXFP4_SWIGLU, 32, 16),
                                      (W.MXFP4_SWIGLU, 2048, 64)])
def test_align_workload_routing(name, M, B):
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, M)
    _check(inp.topk_ids, wl.expert_start, wl.n_local, B)


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("B", [1, 7, 16, 256])
def test_align_random_slices(seed, B):
    rng = np.random.default_rng(seed)
    M, k = int(rng.integers(1, 700)), int(rng.integers(1, 9))
    n_local = int(rng.integers(1, 300))
    start = int(rng.integers(0, 50))
    ids = rng.integers(-5, start + n_local + 40, size=(M, k)).astype(np.int32)  # includes junk ids
    _check(ids, start, n_local, B)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("B", [1, 16, 64, 256])
def test_align_small_batches(seed, B):
    # up to 64 slots: junk and repeated ids, up to 512 local experts, block sizes 1..256
    rng = np.random.default_rng(100 + seed)
    M, k = int(rng.integers(1, 9)), int(rng.integers(1, 9))
    n_local = int(rng.choice([1, 5, 32, 128, 512]))
    start = int(rng.integers(0, 50))
    ids = rng.integers(-5, start + n_local + 40, size=(M, k)).astype(np.int32)
    _check(ids, start, n_local, B)
    _check(np.full((1, 8), start, np.int32), start, n_local, B)   # one expert, all slots


def test_align_edge_cases():
    _check(np.zeros((0, 8), np.int32), 0, 32, 16)                        # no tokens
    _check(np.full((37, 4), 1000, np.int32), 0, 128, 16)                 # everything off-slice
    _check(np.full((300, 2), 5, np.int32), 5, 1, 64)                     # one expert
    rng = np.random.default_rng(9)
    _check(rng.integers(0, 1024, (513, 8)).astype(np.int32), 256, 512, 32)   # largest n_local
    _check(rng.integers(0, 256, (16384, 8)).astype(np.int32), 0, 32, 128)    # 131072 slots


def test_align_several_workgroups_edge_cases():
    rng = np.random.default_rng(11)
    _check(np.full((5000, 2), 7, np.int32), 7, 1, 64)                         # one expert, 5 spans
    _check(rng.integers(100, 300, (3000, 4)).astype(np.int32), 0, 64, 16)     # all off-slice
    _check(rng.integers(0, 40, (1024, 8)).astype(np.int32), 0, 32, 128)       # 8192 = 4 spans exactly
    ids = rng.integers(0, 32, (4097, 2)).astype(np.int32)
    ids[:2048] = 40                                                           # first span all off-slice
    _check(ids, 0, 32, 32)


def test_align_deterministic_and_optional_slot_ids():
    inp = W.make_inputs(W.WORKLOADS[W.NVFP4_ZIPF], 4096)
    a = _run(inp.topk_ids, 0, 32, 128)
    b = _run(inp.topk_ids, 0, 32, 128, slot_ids=False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2] and b[3] is None


@pytest.mark.parametrize("M,k,n_local,B,seed", [
    (4097, 1, 33, 16, 1),      # just above one workgroup's batch: spans of 2048, 2048 and 1
    (2049, 4, 64, 7, 2),       # five spans, the wave-0 scan (64 experts), an odd block size
    (1025, 8, 65, 128, 3),     # the segmented scan (65 experts)
    (20000, 8, 512, 1, 4),     # 79 spans, the largest expert count, block size 1
    (30000, 6, 300, 256, 5),   # 88 spans, the largest block size
    (75000, 8, 32, 128, 6),    # 600000 slots: the workgroup cap, 256 spans of 2344
])
def test_align_several_workgroups(M, k, n_local, B, seed):
    # batches above 4096 slots are split over workgroups that each count the whole batch: the
    # result must be the single sorted order, with skewed routing (a few hot experts) and junk ids
    rng = np.random.default_rng(seed)
    start = int(rng.integers(0, 40))
    p = (np.arange(n_local + 60) + 1.0) ** -1.1
    ids = (rng.choice(n_local + 60, size=(M, k), p=p / p.sum()) + start - 10).astype(np.int32)
    _check(ids, start, n_local, B)
