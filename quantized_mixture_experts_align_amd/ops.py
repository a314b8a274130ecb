"""Torch-tensor wrappers of the C ABI, one per entry point and with the same names.

Argument marshalling only: tensors are checked for device/dtype/contiguity, outputs are
allocated with torch when not given, and every computation runs in libmoe_w4a16.  Streams
are torch's current stream.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib as L


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, dtype, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def align_capacity(M: int, top_k: int, n_local: int, block_m: int):
    s, b = C.c_int64(), C.c_int64()
    L.check(L.lib().moe_align_capacity(M, top_k, n_local, block_m, C.byref(s), C.byref(b)),
            "moe_align_capacity")
    return s.value, b.value


def choose_block_m(numel: int, n_local: int, expected_live: int = 0, K: int = 0) -> int:
    """block_m for the align: numel = M * top_k, expected_live = slots expected on this slice
    (0: all), K = the gate/up reduction length (0: unknown)."""
    b = C.c_int32()
    L.check(L.lib().moe_choose_block_m(numel, n_local, expected_live, K, C.byref(b)), "moe_choose_block_m")
    return b.value


def moe_align(topk_ids: torch.Tensor, expert_start: int, n_local: int, block_m: int,
              slot_local_ids: bool = True, out=None, schedule: Optional[torch.Tensor] = None):
    """-> (sorted_token_ids, expert_ids, num_tokens_post_padded, slot_local_ids or None).
    With `schedule` (int32 [blocks_len]) the call is moe_align_sched, which also writes the MFMA
    GEMM's block schedule there (pass it on as gemm_config(..., block_order=schedule))."""
    _need(topk_ids, torch.int32, "topk_ids")
    M, k = topk_ids.shape
    s_len, b_len = align_capacity(M, k, n_local, block_m)
    dev = topk_ids.device
    if out is None:
        out = (torch.empty(s_len, dtype=torch.int32, device=dev),
               torch.empty(b_len, dtype=torch.int32, device=dev),
               torch.empty(1, dtype=torch.int32, device=dev),
               torch.empty((M, k), dtype=torch.int32, device=dev) if slot_local_ids else None)
    sorted_ids, eids, ntpp, loc = out
    if schedule is None:
        L.check(L.lib().moe_align(_ptr(topk_ids), M, k, expert_start, n_local, block_m, _ptr(sorted_ids),
                                  _ptr(eids), _ptr(ntpp), _ptr(loc), _stream()), "moe_align")
    else:
        _need(schedule, torch.int32, "schedule")
        if schedule.numel() < b_len:
            raise ValueError(f"schedule holds {schedule.numel()} entries, need {b_len}")
        L.check(L.lib().moe_align_sched(_ptr(topk_ids), M, k, expert_start, n_local, block_m, _ptr(sorted_ids),
                                        _ptr(eids), _ptr(ntpp), _ptr(loc), _ptr(schedule), _stream()),
                "moe_align_sched")
    return sorted_ids, eids, ntpp, loc


@dataclass
class PreparedWeights:
    """Device buffer written by moe_w4a16_prepare and the descriptor pointing into it."""
    buffer: torch.Tensor
    desc: L.MoeWeights

    @property
    def N(self) -> int:
        return self.desc.N

    @property
    def K(self) -> int:
        return self.desc.K

    @property
    def n_experts(self) -> int:
        return self.desc.n_experts

    @property
    def weight_bytes(self) -> int:
        return self.buffer.numel()


def prepared_size(qtype: str, E: int, N: int, K: int, flags: int, has_bias: bool):
    n, k, b = C.c_int32(), C.c_int32(), C.c_size_t()
    L.check(L.lib().moe_w4a16_prepared_size(L.QTYPE[qtype], E, N, K, flags, int(has_bias),
                                            C.byref(n), C.byref(k), C.byref(b)),
            "moe_w4a16_prepared_size")
    return n.value, k.value, b.value


def moe_w4a16_prepare(qtype: str, codes: torch.Tensor, scales: torch.Tensor,
                      global_scale: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                      flags: int = 0, zeros: Optional[torch.Tensor] = None,
                      g_idx: Optional[torch.Tensor] = None) -> PreparedWeights:
    """Repack canonical [E, N, K/2] codes and [E, N, K/g] scales (and the [E, N, K/128] zero
    points: uint8 for int4zp_g128, float16 (or its int16 bit patterns) for int4zpf_g128; for
    act-order int4, the int32 [E, K] g_idx, which sets MOE_PREP_ACT_ORDER) into the tiled layout."""
    if g_idx is not None:
        _need(g_idx, torch.int32, "g_idx")
        flags |= L.PREP_ACT_ORDER
    _need(codes, torch.uint8, "codes")
    if not scales.is_cuda or not scales.is_contiguous():
        raise ValueError("scales must be a contiguous device tensor")
    E, N, Kh = codes.shape
    K = Kh * 2
    if global_scale is not None:
        _need(global_scale, torch.float32, "global_scale")
    if bias is not None:
        if bias.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
            raise ValueError("bias must hold bf16 values")
        if not bias.is_cuda or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous device tensor")
    if zeros is not None:
        if qtype == "int4zpf_g128":
            if zeros.dtype not in (torch.float16, torch.int16, torch.uint16):
                raise ValueError("int4zpf_g128 zero points must be float16 values or their bit patterns")
            if not zeros.is_cuda or not zeros.is_contiguous():
                raise ValueError("zeros must be a contiguous device tensor")
        else:
            _need(zeros, torch.uint8, "zeros")
    _, _, nbytes = prepared_size(qtype, E, N, K, flags, bias is not None)
    buf = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    desc = L.MoeWeights()
    L.check(L.lib().moe_w4a16_prepare(L.QTYPE[qtype], _ptr(codes), _ptr(scales), _ptr(global_scale),
                                      _ptr(bias), _ptr(zeros), _ptr(g_idx), E, N, K, flags, _ptr(buf), nbytes,
                                      C.byref(desc),
                                      _stream()), "moe_w4a16_prepare")
    return PreparedWeights(buf, desc)


def moe_permute_cols(src: torch.Tensor, W: PreparedWeights, slot_expert: torch.Tensor, row_div: int,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Rows of A for a GEMM on act-order weights W: out[r, j] = src[r // row_div, perm_e[j]] for
    every slot r (= len(slot_expert)) routed to a local expert e; other rows are not written."""
    if not src.is_cuda or src.dtype != torch.bfloat16 or src.dim() != 2 or src.stride(1) != 1:
        raise ValueError("src must be a bf16 device matrix with unit column stride")
    _need(slot_expert, torch.int32, "slot_expert")
    if not W.desc.perm:
        raise ValueError("moe_permute_cols: the weights were prepared without act-order")
    rows, K = slot_expert.numel(), W.K
    if out is None:
        out = torch.empty((rows, K), dtype=torch.bfloat16, device=src.device)
    _need(out, torch.bfloat16, "out")
    L.check(L.lib().moe_permute_cols(_ptr(src), src.stride(0), row_div, W.desc.perm, K, W.n_experts,
                                     _ptr(slot_expert), rows, _ptr(out), out.stride(0), _stream()),
            "moe_permute_cols")
    return out


def moe_norm_weight(w: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _need(w, torch.bfloat16, "post_norm_w")
    out = torch.empty_like(w) if out is None else out
    L.check(L.lib().moe_norm_weight(_ptr(w), w.numel(), _ptr(out), _stream()), "moe_norm_weight")
    return out


def gemm_config(kernel: int = L.GEMM_AUTO, ng: int = 0, ksplit: int = 0, gemv_rows: int = 0,
                group_m: int = 0, block_order=None):
    """block_order: the schedule tensor moe_align(..., schedule=) filled, or its device address
    (the tensor must outlive every launch that uses the configuration)."""
    if isinstance(block_order, torch.Tensor):
        _need(block_order, torch.int32, "block_order")
        block_order = block_order.data_ptr()
    return L.MoeGemmConfig(kernel, ng, ksplit, gemv_rows, group_m, block_order)


def gemm_choose(W: PreparedWeights, numel: int, block_m: int, num_cus: int = 0,
                resident: Optional[tuple] = None) -> L.MoeGemmConfig:
    """Launch configuration; `resident` = MFMA workgroups per CU at 1, 2, 4 tiles per wave
    (moe_gemm_choose_occ), else the current device's (moe_gemm_choose)."""
    c = L.MoeGemmConfig()
    if resident is None:
        L.check(L.lib().moe_gemm_choose(C.byref(W.desc), numel, block_m, num_cus, C.byref(c)),
                "moe_gemm_choose")
    else:
        r = (C.c_int32 * 3)(*resident)
        L.check(L.lib().moe_gemm_choose_occ(C.byref(W.desc), numel, block_m, num_cus, C.byref(r), C.byref(c)),
                "moe_gemm_choose_occ")
    return c


def gemm_occupancy(W: PreparedWeights, block_m: int, gated: bool) -> tuple:
    """(resident workgroups per CU at 1, 2, 4 tiles per wave) of the MFMA kernel, from the HIP
    occupancy API on the current device."""
    r = (C.c_int32 * 3)()
    L.check(L.lib().moe_gemm_occupancy(C.byref(W.desc), block_m, int(gated), C.byref(r)), "moe_gemm_occupancy")
    return tuple(r)


def moe_w4a16_gemm(A: torch.Tensor, W: PreparedWeights, sorted_token_ids: torch.Tensor,
                   expert_ids: torch.Tensor, num_tokens_post_padded: torch.Tensor, numel: int,
                   top_k: int, block_m: int, out: Optional[torch.Tensor] = None,
                   cfg: Optional[L.MoeGemmConfig] = None) -> torch.Tensor:
    """C[slot] = dequant(W[e]) . A[slot // top_k] (+ bias) for the live slots; C is [numel, N]."""
    _need(A, torch.bfloat16, "A")
    if out is None:
        out = torch.empty((numel, W.N), dtype=torch.bfloat16, device=A.device)
    _need(out, torch.bfloat16, "out")
    L.check(L.lib().moe_w4a16_gemm(_ptr(A), A.shape[0], A.stride(0), _ptr(out), out.stride(0),
                                   C.byref(W.desc), _ptr(sorted_token_ids), _ptr(expert_ids),
                                   _ptr(num_tokens_post_padded), numel, top_k, block_m,
                                   None if cfg is None else C.byref(cfg), _stream()),
            "moe_w4a16_gemm")
    return out


def moe_w4a16_gemm_act(kind: str, A: torch.Tensor, W13: PreparedWeights, sorted_token_ids: torch.Tensor,
                       expert_ids: torch.Tensor, num_tokens_post_padded: torch.Tensor, numel: int,
                       top_k: int, block_m: int, alpha: float = 1.702, limit: float = float("inf"),
                       out: Optional[torch.Tensor] = None,
                       cfg: Optional[L.MoeGemmConfig] = None) -> torch.Tensor:
    """out[slot] = act(gate, up) of the gate/up GEMM (or relu(h)^2 of the non-gated GEMM1),
    fused into one launch; out is [numel, I]."""
    _need(A, torch.bfloat16, "A")
    if out is None:
        I = W13.N if kind == "relu2" else W13.N // 2
        out = torch.empty((numel, I), dtype=torch.bfloat16, device=A.device)
    _need(out, torch.bfloat16, "out")
    L.check(L.lib().moe_w4a16_gemm_act(L.ACT[kind], alpha, limit, _ptr(A), A.shape[0], A.stride(0),
                                       _ptr(out), out.stride(0), C.byref(W13.desc),
                                       _ptr(sorted_token_ids), _ptr(expert_ids),
                                       _ptr(num_tokens_post_padded), numel, top_k, block_m,
                                       None if cfg is None else C.byref(cfg), _stream()),
            "moe_w4a16_gemm_act")
    return out


FUSED_ALIGN_SLOTS = 128  # most slots (M * top_k) of moe_w4a16_gemm_act_routed


def moe_w4a16_gemm_act_routed(kind: str, A: torch.Tensor, W13: PreparedWeights, topk_ids: torch.Tensor,
                              expert_start: int, block_m: int, alpha: float = 1.702,
                              limit: float = float("inf"), out: Optional[torch.Tensor] = None,
                              align_out=None, cfg: Optional[L.MoeGemmConfig] = None):
    """moe_align + moe_w4a16_gemm_act in one launch for at most 128 slots (block_m <= 16).
    -> (out, (sorted_token_ids, expert_ids, num_tokens_post_padded, slot_local_ids))."""
    _need(A, torch.bfloat16, "A")
    _need(topk_ids, torch.int32, "topk_ids")
    M, k = topk_ids.shape
    n_local = W13.desc.n_experts
    dev = topk_ids.device
    if align_out is None:
        s_len, b_len = align_capacity(M, k, n_local, block_m)
        align_out = (torch.empty(s_len, dtype=torch.int32, device=dev),
                     torch.empty(b_len, dtype=torch.int32, device=dev),
                     torch.empty(1, dtype=torch.int32, device=dev),
                     torch.empty((M, k), dtype=torch.int32, device=dev))
    sorted_ids, eids, ntpp, loc = align_out
    if out is None:
        I = W13.N if kind == "relu2" else W13.N // 2
        out = torch.empty((M * k, I), dtype=torch.bfloat16, device=A.device)
    _need(out, torch.bfloat16, "out")
    L.check(L.lib().moe_w4a16_gemm_act_routed(L.ACT[kind], alpha, limit, _ptr(A), A.shape[0], A.stride(0),
                                              _ptr(out), out.stride(0), C.byref(W13.desc), _ptr(topk_ids),
                                              M, k, expert_start, block_m, _ptr(sorted_ids), _ptr(eids),
                                              _ptr(ntpp), _ptr(loc), None if cfg is None else C.byref(cfg),
                                              _stream()),
            "moe_w4a16_gemm_act_routed")
    return out, align_out


def moe_act(kind: str, h: torch.Tensor, I: int, slot_local_ids: Optional[torch.Tensor] = None,
            alpha: float = 1.702, limit: float = float("inf"),
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _need(h, torch.bfloat16, "h")
    R = h.shape[0]
    if out is None:
        out = torch.empty((R, I), dtype=torch.bfloat16, device=h.device)
    L.check(L.lib().moe_act(L.ACT[kind], _ptr(h), h.stride(0), _ptr(out), out.stride(0), R, I,
                            _ptr(slot_local_ids), alpha, limit, _stream()), "moe_act")
    return out


def combine_counters(M: int, W: PreparedWeights, device) -> torch.Tensor:
    """Zeroed arrival counters for moe_w4a16_gemm_combine (M * N / 16, enough for every ng); every
    completed call leaves them zero, so one buffer serves calls of up to M tokens in turn."""
    return torch.zeros(max(1, M * (W.N // 16)), dtype=torch.int32, device=device)


def moe_w4a16_gemm_combine(A: torch.Tensor, W: PreparedWeights, sorted_token_ids: torch.Tensor,
                           expert_ids: torch.Tensor, num_tokens_post_padded: torch.Tensor,
                           topk_weights: torch.Tensor, slot_local_ids: torch.Tensor, block_m: int,
                           counters: torch.Tensor, y: torch.Tensor, out: Optional[torch.Tensor] = None,
                           routed_scaling_factor: float = 1.0,
                           cfg: Optional[L.MoeGemmConfig] = None) -> torch.Tensor:
    """Down GEMM (A row = slot) with the no-norm top-k weighted sum fused in: y[slot] as
    moe_w4a16_gemm, out[t] = rsf * sum_s g[t, s] * y[t * k + s] over live slots; out is [M, N]."""
    _need(A, torch.bfloat16, "A")
    _need(y, torch.bfloat16, "y")
    _need(topk_weights, torch.float32, "topk_weights")
    _need(slot_local_ids, torch.int32, "slot_local_ids")
    _need(counters, torch.int32, "counters")
    M, k = topk_weights.shape
    if out is None:
        out = torch.empty((M, W.N), dtype=torch.bfloat16, device=A.device)
    _need(out, torch.bfloat16, "out")
    L.check(L.lib().moe_w4a16_gemm_combine(_ptr(A), A.shape[0], A.stride(0), _ptr(y), y.stride(0),
                                           C.byref(W.desc), _ptr(sorted_token_ids), _ptr(expert_ids),
                                           _ptr(num_tokens_post_padded), M, k, block_m, _ptr(topk_weights),
                                           _ptr(slot_local_ids), routed_scaling_factor, _ptr(counters),
                                           counters.numel(), _ptr(out), out.stride(0),
                                           None if cfg is None else C.byref(cfg), _stream()),
            "moe_w4a16_gemm_combine")
    return out


def moe_w4a16_gemm_combine_noalloc(A: torch.Tensor, W: PreparedWeights, sorted_token_ids: torch.Tensor,
                                   expert_ids: torch.Tensor, num_tokens_post_padded: torch.Tensor,
                                   topk_weights: torch.Tensor, slot_local_ids: torch.Tensor, block_m: int,
                                   y: torch.Tensor, out: torch.Tensor, routed_scaling_factor: float = 1.0,
                                   cfg: Optional[L.MoeGemmConfig] = None) -> torch.Tensor:
    """moe_w4a16_gemm_combine with its arrival counters in the library's scratch memory (no
    caller workspace, nothing allocated: `y` and `out` must be given)."""
    _need(A, torch.bfloat16, "A")
    _need(y, torch.bfloat16, "y")
    _need(out, torch.bfloat16, "out")
    _need(topk_weights, torch.float32, "topk_weights")
    _need(slot_local_ids, torch.int32, "slot_local_ids")
    M, k = topk_weights.shape
    L.check(L.lib().moe_w4a16_gemm_combine_noalloc(_ptr(A), A.shape[0], A.stride(0), _ptr(y), y.stride(0),
                                                   C.byref(W.desc), _ptr(sorted_token_ids), _ptr(expert_ids),
                                                   _ptr(num_tokens_post_padded), M, k, block_m,
                                                   _ptr(topk_weights), _ptr(slot_local_ids),
                                                   routed_scaling_factor, _ptr(out), out.stride(0),
                                                   None if cfg is None else C.byref(cfg), _stream()),
            "moe_w4a16_gemm_combine_noalloc")
    return out


def moe_combine(y: torch.Tensor, topk_weights: torch.Tensor, slot_local_ids: torch.Tensor,
                norm_w: Optional[torch.Tensor] = None, eps: float = 1e-8,
                out: Optional[torch.Tensor] = None, routed_scaling_factor: float = 1.0) -> torch.Tensor:
    _need(y, torch.bfloat16, "y")
    _need(topk_weights, torch.float32, "topk_weights")
    _need(slot_local_ids, torch.int32, "slot_local_ids")
    M, k = topk_weights.shape
    H = y.shape[-1]
    if out is None:
        out = torch.empty((M, H), dtype=torch.bfloat16, device=y.device)
    L.check(L.lib().moe_combine(_ptr(y), _ptr(topk_weights), _ptr(slot_local_ids), _ptr(norm_w), eps,
                                routed_scaling_factor, M, k, H, _ptr(out), _stream()), "moe_combine")
    return out


def requant_choose(E: int, max_m: int, K: int, expected_rows: int = 0, num_cus: int = 0) -> L.MoeRequantConfig:
    """Launch hint for moe_fp8_requant; expected_rows = live rows per expert if known (0 = not)."""
    c = L.MoeRequantConfig()
    if num_cus <= 0:
        num_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    L.check(L.lib().moe_fp8_requant_choose(E, max_m, K, expected_rows, num_cus, C.byref(c)),
            "moe_fp8_requant_choose")
    return c


def requant_config(workgroups: int, unroll: int) -> L.MoeRequantConfig:
    return L.MoeRequantConfig(workgroups, unroll)


def moe_fp8_requant(x: torch.Tensor, scales: torch.Tensor, masked_m: torch.Tensor,
                    tensor_scale: torch.Tensor, group_size: int = 128,
                    out: Optional[torch.Tensor] = None,
                    cfg: Optional[L.MoeRequantConfig] = None) -> torch.Tensor:
    """x uint8 [E, max_m, K] (float8 e4m3fn codes; a float8_e4m3fn tensor is viewed as bytes);
    scales float32 [E, max_m, K/group_size], any strides (a transposed view of a column-major
    [E, K/group_size, max_m] array is passed as is); masked_m int32 [E]; tensor_scale float32 [1].
    Returns out (uint8, same shape as x): live rows requantised, other rows untouched."""
    if x.dtype == torch.float8_e4m3fn:
        x = x.view(torch.uint8)
    _need(x, torch.uint8, "x")
    _need(masked_m, torch.int32, "masked_m")
    _need(tensor_scale, torch.float32, "tensor_scale")
    if not scales.is_cuda or scales.dtype != torch.float32 or scales.dim() != 3:
        raise ValueError("scales must be a float32 device tensor [E, max_m, K/group_size]")
    E, max_m, K = x.shape
    if tuple(scales.shape) != (E, max_m, K // group_size) or tuple(masked_m.shape) != (E,):
        raise ValueError(f"shapes: x {tuple(x.shape)}, scales {tuple(scales.shape)}, "
                         f"masked_m {tuple(masked_m.shape)} do not match group_size {group_size}")
    if out is None:
        out = torch.empty_like(x)
    elif out.dtype == torch.float8_e4m3fn:
        out = out.view(torch.uint8)
    _need(out, torch.uint8, "out")
    if tuple(out.shape) != tuple(x.shape):
        raise ValueError(f"out {tuple(out.shape)} must have the shape of x {tuple(x.shape)}")
    se, sm, sg = scales.stride()
    L.check(L.lib().moe_fp8_requant(_ptr(x), _ptr(scales), se, sm, sg, _ptr(masked_m), _ptr(tensor_scale),
                                    E, max_m, K, group_size, _ptr(out),
                                    None if cfg is None else C.byref(cfg), _stream()),
            "moe_fp8_requant")
    return out
