"""GPU parity of moe_fp8_requant (float8 per-token-group -> per-tensor requant) against the CPU
oracle: bit-exact bytes in every live row, every other row slot untouched, for the requant
workloads at full size, both scale layouts, saturating tensor scales, every float8 code
(NaN codes included), ties decided by the float32 products, ragged K, other group sizes, up to
1024 experts, clamped row counts, in place, and every launch geometry."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import requant as R
from tests.gpu_util import announce

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t if dtype is None else t.to(dtype)


def _run(x, scales, masked_m, ts, group=128, cfg=None, col_major=False, inplace=False):
    """Requant on the GPU; returns the whole output array (uint8 [E, max_m, K])."""
    from quantized_mixture_experts_align_amd import moe_fp8_requant
    E, max_m, K = x.shape
    xd = _dev(x)
    if col_major:   # stored [E, G, max_m], passed as the [E, max_m, G] view
        sd = _dev(np.transpose(scales, (0, 2, 1))).transpose(1, 2)
        assert not sd.is_contiguous()
    else:
        sd = _dev(scales)
    md = _dev(np.asarray(masked_m, dtype=np.int32))
    td = torch.tensor([ts], dtype=torch.float32, device="cuda")
    if inplace:
        out = xd
    else:
        out = torch.full_like(xd, SENTINEL)
    moe_fp8_requant(xd, sd, md, td, group_size=group, out=out, cfg=cfg)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(x, scales, masked_m, ts, group=128, **kw):
    got = _run(x, scales, masked_m, ts, group, **kw)
    want, live = R.requant(x, scales, masked_m, np.float32(ts), group)
    bad = np.argwhere((got != want) & live[..., None])
    assert bad.size == 0, (f"{len(bad)} live bytes differ; first at {tuple(bad[0])}: "
                           f"got {got[tuple(bad[0])]:#04x} want {want[tuple(bad[0])]:#04x}")
    untouched = x if kw.get("inplace") else np.full_like(x, SENTINEL)
    assert np.array_equal(got[~live], untouched[~live]), "a row slot that is not live was written"
    return got, live


@pytest.mark.parametrize("name", list(W.REQUANT_WORKLOADS))
@pytest.mark.parametrize("col_major", [False, True])
def test_workloads_full_size(name, col_major):
    wl = W.REQUANT_WORKLOADS[name]
    inp = W.requant_inputs_for(wl)
    announce(f"requant {name} col_major={col_major} E={wl.E} max_m={inp.x.shape[1]} K={wl.K}")
    got, live = _check(inp.x, inp.scales, inp.masked_m, inp.tensor_scale, col_major=col_major)
    assert live.sum() == int(W.requant_counts(wl).sum())


@pytest.mark.parametrize("factor", [0.25, 1.0, 3.0])
def test_saturating_and_small_tensor_scales(factor):
    inp = W.make_requant_inputs(16, 9, 1024, np.arange(16) % 10, seed=31, tensor_scale_factor=factor)
    got, live = _check(inp.x, inp.scales, inp.masked_m, inp.tensor_scale)
    if factor < 1:
        assert (got[live] & 0x7F == 0x7E).any()     # saturated to +-448


def test_every_code_with_wide_scales():
    # each live row holds all 256 codes (NaN codes 0x7F / 0xFF included) in a different order;
    # scales span 2^-30 .. 2^30 (float8 subnormals, zeros and saturation), zero and negative
    E, max_m, K = 4, 8, 2048
    x = np.stack([np.stack([np.roll(np.tile(np.arange(256), K // 256), 37 * (e * max_m + m))
                            for m in range(max_m)]) for e in range(E)]).astype(np.uint8)
    rng = np.random.default_rng(17)
    scales = (np.exp2(rng.uniform(-30, 30, size=(E, max_m, K // 128)))
              * rng.choice([1.0, -1.0], size=(E, max_m, K // 128))).astype(np.float32)
    scales[0, 0, :3] = [0.0, -0.0, 1.0]
    for ts in (1.0, 0.0123, 1e-20):
        got, live = _check(x, scales, [8, 7, 1, 5], ts)
    assert (got[live] == 0x7F).any() and (got[live] == 0x80).any()


@pytest.mark.parametrize("ts", [1.0, 0.0, -0.0, float("inf"), float("nan"), 3.0e-39])
def test_degenerate_scales(ts):
    # infinite, NaN, zero and huge group scales, and tensor scales whose reciprocal is infinite,
    # zero or NaN: inf * 0 and NaN products must still give 0x7F, overflow saturates
    rng = np.random.default_rng(23)
    E, max_m, K = 3, 4, 1024
    x = rng.integers(0, 256, size=(E, max_m, K), dtype=np.uint8)
    x[0, 0, :4] = [0x00, 0x80, 0x7F, 0xFF]
    scales = np.exp2(rng.uniform(-4, 4, size=(E, max_m, K // 128))).astype(np.float32)
    special = np.array([np.inf, -np.inf, np.nan, 0.0, -0.0, 3.0e38, 1e-45, -2.5], np.float32)
    scales[0, 0, :] = special
    scales[1, :, 3] = special[:max_m]
    got, live = _check(x, scales, [4, 3, 2], ts)
    assert (got[live] == 0x7F).any()


def test_float32_products_decide_ties():
    # x * s one half float32 ulp above an e4m3 midpoint rounds onto it in float32, then to the
    # even code: the kernel must take the two float32 roundings, not an exact or fused product
    pos = R.decode_e4m3fn(np.arange(0x7F))
    mids = ((pos[1:] + pos[:-1]) / 2)[8:100]
    cand = []
    for xv in pos[40:90]:
        for mv in mids:
            s32 = np.float32(mv / xv)
            if np.float32(xv) * s32 == np.float32(mv) and np.float64(xv) * np.float64(s32) > mv:
                cand.append((xv, s32))
    cand = cand[:128]
    n = len(cand)
    x = np.repeat(R.encode_e4m3fn_sat(np.array([c[0] for c in cand]))[:, None], 128, axis=1)[None]
    scales = np.array([c[1] for c in cand], dtype=np.float32)[None, :, None]
    _check(x, scales, [n], 1.0)


@pytest.mark.parametrize("K,group", [(128, 128), (384, 128), (1152, 128), (7168, 128), (1040, 16),
                                     (960, 64), (3072, 32)])
def test_ragged_k_and_group_sizes(K, group):
    # K not a multiple of the 1024-byte work item; random codes (NaN codes included) and one
    # random scale per (row, group)
    E, max_m = 5, 7
    rng = np.random.default_rng(K + group)
    x = rng.integers(0, 256, size=(E, max_m, K), dtype=np.uint8)
    scales = np.exp2(rng.uniform(-6, 6, size=(E, max_m, K // group))).astype(np.float32)
    _check(x, scales, [7, 0, 3, 9, -2], 1.5, group)


@pytest.mark.parametrize("E", [1, 63, 64, 65, 256, 257, 1000, 1024])
def test_expert_counts_and_clamped_rows(E):
    # row counts include negatives and values above max_m (clamped), many empty experts
    rng = np.random.default_rng(E)
    max_m = 3
    mm = rng.integers(-2, 6, size=E).astype(np.int32)
    inp = W.make_requant_inputs(E, max_m, 256, mm, seed=E)
    _check(inp.x, inp.scales, mm, inp.tensor_scale)


def test_no_live_rows_and_empty_shapes():
    inp = W.make_requant_inputs(40, 4, 512, np.zeros(40, np.int32), seed=3)
    got, live = _check(inp.x, inp.scales, inp.masked_m, inp.tensor_scale)
    assert not live.any()
    # E = 0 and max_m = 0 launch nothing and succeed
    for E, max_m in ((0, 4), (3, 0)):
        x = np.zeros((E, max_m, 256), np.uint8)
        got = _run(x, np.zeros((E, max_m, 2), np.float32), np.zeros(E, np.int32), 1.0)
        assert got.shape == x.shape


def test_in_place():
    inp = W.make_requant_inputs(8, 6, 1024, [6, 1, 0, 3, 6, 2, 5, 4], seed=9)
    _check(inp.x, inp.scales, inp.masked_m, inp.tensor_scale, inplace=True)


def test_results_do_not_depend_on_the_launch_geometry():
    from quantized_mixture_experts_align_amd import requant_config
    wl = W.REQUANT_WORKLOADS["requant_e32_k7168_rows32_skew16"]
    inp = W.make_requant_inputs(32, 40, 3072, W.requant_counts(wl) // 13, seed=21)
    ref = _run(inp.x, inp.scales, inp.masked_m, inp.tensor_scale)
    want, live = R.requant(inp.x, inp.scales, inp.masked_m, inp.tensor_scale)
    assert np.array_equal(ref[live], want[live])
    for wg, u in [(1, 1), (1, 4), (3, 2), (7, 1), (64, 4), (512, 2), (4096, 1)]:
        got = _run(inp.x, inp.scales, inp.masked_m, inp.tensor_scale, cfg=requant_config(wg, u))
        assert np.array_equal(got, ref), (wg, u)


def test_graph_replays_on_new_inputs():
    # one launch captured in a HIP graph, replayed on three different batches copied into the same
    # buffers, with eager work between the replays: every replay equals the oracle
    from quantized_mixture_experts_align_amd import moe_fp8_requant
    E, max_m, K = 24, 6, 2048
    x = torch.empty((E, max_m, K), dtype=torch.uint8, device="cuda")
    sc = torch.empty((E, max_m, K // 128), dtype=torch.float32, device="cuda")
    mm = torch.empty(E, dtype=torch.int32, device="cuda")
    ts = torch.empty(1, dtype=torch.float32, device="cuda")
    out = torch.full_like(x, SENTINEL)
    batches = []
    for seed in range(4):
        rng = np.random.default_rng(100 + seed)
        inp = W.make_requant_inputs(E, max_m, K, rng.integers(0, max_m + 1, size=E), seed=100 + seed)
        batches.append(inp)
    def load(inp):
        x.copy_(torch.from_numpy(inp.x)); sc.copy_(torch.from_numpy(inp.scales))
        mm.copy_(torch.from_numpy(inp.masked_m)); ts.fill_(float(inp.tensor_scale))
        out.fill_(SENTINEL)
    load(batches[0])
    moe_fp8_requant(x, sc, mm, ts, out=out)          # eager warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe_fp8_requant(x, sc, mm, ts, out=out)
    for inp in batches[1:]:
        load(inp)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        want, live = R.requant(inp.x, inp.scales, inp.masked_m, inp.tensor_scale)
        assert np.array_equal(got[live], want[live])
        assert (got[~live] == SENTINEL).all()


def test_rejects_bad_arguments():
    from quantized_mixture_experts_align_amd import moe_fp8_requant, requant_config
    x = torch.zeros((2, 3, 256), dtype=torch.uint8, device="cuda")
    s = torch.ones((2, 3, 2), dtype=torch.float32, device="cuda")
    m = torch.ones(2, dtype=torch.int32, device="cuda")
    t = torch.ones(1, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        moe_fp8_requant(x, s, m, t, cfg=requant_config(0, 1))
    with pytest.raises(ValueError):
        moe_fp8_requant(x, s, m, t, cfg=requant_config(4, 3))
    with pytest.raises(ValueError):
        moe_fp8_requant(x, torch.ones((2, 3, 32), dtype=torch.float32, device="cuda"), m, t, group_size=8)
    flat = torch.zeros(2 * 3 * 256 + 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):   # out overlapping x without being x
        moe_fp8_requant(flat[:1536].view(2, 3, 256), s, m, t, out=flat[16:].view(2, 3, 256))
