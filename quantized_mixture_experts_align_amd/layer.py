"""The expert layer as the five C-ABI calls: align -> GEMM1 -> act -> GEMM2 -> combine.

Everything runs on torch's current stream without host synchronisation, so a forward can be
captured in a HIP graph when a Workspace is passed (no allocation inside).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib as L
from . import ops


@dataclass
class Workspace:
    """Buffers of one forward for M tokens.  The GEMM1 output h [numel, 2I] and the GEMM2
    output y [numel, H] share one allocation (h is dead once the activation has run), the
    same plan as the experiment's cache13."""
    M: int
    block_m: int
    sorted_ids: torch.Tensor
    expert_ids: torch.Tensor
    ntpp: torch.Tensor
    slot_local: torch.Tensor
    buf13: torch.Tensor
    a: torch.Tensor
    out: torch.Tensor
    cfgs: Optional[tuple] = None    # (gate/up, down) GEMM launch configurations
    perm: Optional[torch.Tensor] = None   # act-order: the gathered A of a GEMM [numel, max(H, I)]
    counters: Optional[torch.Tensor] = None  # fused weighted sum: arrival counters, kept zero
    sched: Optional[torch.Tensor] = None  # MFMA GEMMs: the align's block schedule [blocks_len]


class MoELayer:
    """One GPU's slice of a W4A16 MoE expert layer (experts [expert_start, expert_start + n_local)).

    ``w13`` / ``w2``: dicts of device tensors in the canonical layouts: ``codes`` uint8
    [E, N, K/2], ``scales`` [E, N, K/g], optional ``gs`` fp32 [E] (NVFP4), ``bias`` bf16 [E, N],
    ``zeros`` uint8 [E, N, K/128] (asymmetric int4) and ``g_idx`` int32 [E, K] (act-order int4:
    the GEMM then reads its activations gathered into group order by moe_permute_cols).
    ``w13`` has 2I rows (gate, up) for the gated activations and I rows for ``relu2``.
    ``routed_scaling_factor`` multiplies the combined output.
    """

    def __init__(self, qtype: str, w13: dict, w2: dict, *, expert_start: int, n_local: int,
                 top_k: int, act: str = "silu_mul", alpha: float = 1.702,
                 limit: float = float("inf"), post_norm_w: Optional[torch.Tensor] = None,
                 eps: float = 1e-8, interleaved_w13: bool = False, pad: bool = False,
                 n_global: Optional[int] = None, routed_scaling_factor: float = 1.0):
        if act not in L.ACT:
            raise ValueError(f"unknown activation {act!r}")
        self.qtype, self.expert_start, self.n_local, self.top_k = qtype, expert_start, n_local, top_k
        self.n_global = n_global
        self.act, self.alpha, self.limit, self.eps = act, alpha, limit, eps
        self.gated = L.GATED[act]
        self.routed_scaling_factor = routed_scaling_factor
        if self.gated:
            f13 = L.PREP_GATE_UP | (L.PREP_INTERLEAVED if interleaved_w13 else 0) | (L.PREP_PAD if pad else 0)
        else:
            if interleaved_w13:
                raise ValueError("interleaved gate/up rows need a gated activation")
            f13 = L.PREP_PAD if pad else 0
        f2 = L.PREP_PAD if pad else 0
        self.W13 = ops.moe_w4a16_prepare(qtype, w13["codes"], w13["scales"], w13.get("gs"),
                                         w13.get("bias"), f13, w13.get("zeros"), w13.get("g_idx"))
        self.W2 = ops.moe_w4a16_prepare(qtype, w2["codes"], w2["scales"], w2.get("gs"),
                                        w2.get("bias"), f2, w2.get("zeros"), w2.get("g_idx"))
        self.act_order = (bool(self.W13.desc.perm), bool(self.W2.desc.perm))
        self.I = self.W13.N // 2 if self.gated else self.W13.N
        if self.W2.K != self.I:
            raise ValueError(f"down projection K={self.W2.K} != intermediate {self.I}")
        if self.W2.n_experts != n_local or self.W13.n_experts != n_local:
            raise ValueError("weights must hold exactly the n_local local experts")
        self.H = self.W2.N
        self.norm_w = None if post_norm_w is None else ops.moe_norm_weight(post_norm_w)

    def expected_local_slots(self, M: int) -> int:
        """Launch hint: slots expected on this slice (all of them when n_global is unknown).
        Only launch shapes depend on it, never results."""
        numel = M * self.top_k
        if not self.n_global or self.n_global <= self.n_local:
            return numel
        return max(1, -(-numel * self.n_local // self.n_global))

    def block_m(self, M: int) -> int:
        return ops.choose_block_m(M * self.top_k, self.n_local, self.expected_local_slots(M), self.W13.K)

    def configs(self, M: int, block_m: int):
        """GEMM launch configurations (gate/up, down) for a batch of M tokens."""
        hint = self.expected_local_slots(M)
        return ops.gemm_choose(self.W13, hint, block_m), ops.gemm_choose(self.W2, hint, block_m)

    def workspace(self, M: int, block_m: Optional[int] = None, device=None) -> Workspace:
        device = device or self.W13.buffer.device
        B = block_m or self.block_m(M)
        s_len, b_len = ops.align_capacity(M, self.top_k, self.n_local, B)
        numel = M * self.top_k
        i32 = dict(dtype=torch.int32, device=device)
        bf = dict(dtype=torch.bfloat16, device=device)
        perm = None
        if any(self.act_order):
            perm = torch.empty(numel * max(self.W13.K, self.W2.K), **bf)
        cfgs = self.configs(M, B)
        sched = None
        if B > 16 and min(self.W13.K, self.W2.K) >= 2048 and any(c.kernel == L.GEMM_MFMA for c in cfgs):
            # the align writes the MFMA GEMMs' block schedule, the GEMMs take their blocks in it.
            # Only for long K loops: measured on the int4 layers (K = 512 / 1024, 64-slot blocks)
            # the schedule's align work and prologue read cost 1-1.5 us of a 40-75 us step with
            # the GEMMs unchanged; 16-slot blocks all have one 16-slot group (the align order).
            sched = torch.empty(b_len, **i32)
            for c in cfgs:
                if c.kernel == L.GEMM_MFMA:
                    c.block_order = sched.data_ptr()
        return Workspace(M, B, torch.empty(s_len, **i32), torch.empty(b_len, **i32),
                         torch.empty(1, **i32), torch.empty((M, self.top_k), **i32),
                         torch.empty(numel * max(self.W13.N, self.H), **bf),
                         torch.empty((numel, self.I), **bf), torch.empty((M, self.H), **bf),
                         cfgs, perm, sched=sched)

    def _combinable(self, B: int, cfg2) -> bool:
        # the weighted sum fuses into the streaming decode kernel's down GEMM when there is no norm
        return (self.norm_w is None and B <= 16 and cfg2.kernel == L.GEMM_DECODE
                and cfg2.gemv_rows == 0)

    def forward(self, x: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                ws: Optional[Workspace] = None, cfg13=None, cfg2=None,
                fused_act: bool = True, fused_align: Optional[bool] = None,
                fused_combine: bool = False) -> torch.Tensor:
        """align -> gate/up GEMM -> activation -> down GEMM -> combine.  With fused_act the
        activation runs in the GEMM1 epilogue (bitwise the same result, one launch and one
        [numel, N13] round trip less); for a gated activation cfg13 then needs ng 2 or 4.
        With fused_align (default: whenever it applies -- at most 128 slots, the streaming decode
        kernel, fused_act) the align runs inside that same launch as well (bitwise the same).
        With fused_combine (no norm, the streaming decode kernel for the down GEMM) the weighted
        sum runs in the down GEMM's launch (bitwise the same; counters are added to the workspace
        on first use).  It is off by default: measured on MI355X, its cross-XCD release/acquire
        fences cost more than the combine launch they save."""
        M = x.shape[0]
        if ws is None:
            ws = self.workspace(M, device=x.device)
        if ws.M != M:
            raise ValueError(f"workspace is for M={ws.M}, got {M}")
        numel = M * self.top_k
        B = ws.block_m
        if cfg13 is None or cfg2 is None:
            c13, c2 = ws.cfgs if ws.cfgs is not None else self.configs(M, B)
            cfg13 = cfg13 or c13
            cfg2 = cfg2 or c2
        # (act-order gate/up weights need the slots' experts before GEMM1: no fused align)
        routable = (numel <= ops.FUSED_ALIGN_SLOTS and B <= 16 and cfg13.kernel == L.GEMM_DECODE
                    and cfg13.gemv_rows == 0 and not self.act_order[0])
        if fused_align is None:
            fused_align = fused_act and routable
        if fused_align and not (fused_act and routable):
            raise ValueError("fused_align needs fused_act, at most 128 slots, block_m <= 16 and the "
                             "streaming decode kernel")
        align_out = (ws.sorted_ids, ws.expert_ids, ws.ntpp, ws.slot_local)
        if fused_act and self.gated and cfg13.ng < 2:
            cfg13 = ops.gemm_config(cfg13.kernel, 2, cfg13.ksplit, cfg13.gemv_rows, cfg13.group_m,
                                    cfg13.block_order)
        if fused_align and cfg2.block_order:
            # the align fused into GEMM1 writes no schedule: the down GEMM takes the align order
            cfg2 = ops.gemm_config(cfg2.kernel, cfg2.ng, cfg2.ksplit, cfg2.gemv_rows, cfg2.group_m)
        if fused_align:
            _, (sorted_ids, eids, ntpp, loc) = ops.moe_w4a16_gemm_act_routed(
                self.act, x, self.W13, topk_ids, self.expert_start, B, self.alpha, self.limit,
                out=ws.a, align_out=align_out, cfg=cfg13)
        else:
            # (a configuration that names the workspace's schedule gets it written by this align)
            sorted_ids, eids, ntpp, loc = ops.moe_align(topk_ids, self.expert_start, self.n_local, B,
                                                        out=align_out, schedule=ws.sched)
            a1, k1 = x, self.top_k
            if self.act_order[0]:   # one gathered row per slot, read with top_k = 1
                a1 = ops.moe_permute_cols(x, self.W13, loc.view(-1), self.top_k,
                                          out=ws.perm[: numel * self.W13.K].view(numel, self.W13.K))
                k1 = 1
            if fused_act:
                ops.moe_w4a16_gemm_act(self.act, a1, self.W13, sorted_ids, eids, ntpp, numel, k1,
                                       B, self.alpha, self.limit, out=ws.a, cfg=cfg13)
            else:
                h = ws.buf13[: numel * self.W13.N].view(numel, self.W13.N)
                ops.moe_w4a16_gemm(a1, self.W13, sorted_ids, eids, ntpp, numel, k1, B, out=h,
                                   cfg=cfg13)
                ops.moe_act(self.act, h, self.I, loc.view(-1), self.alpha, self.limit, out=ws.a)
        y = ws.buf13[: numel * self.H].view(numel, self.H)
        a2 = ws.a
        if self.act_order[1]:
            a2 = ops.moe_permute_cols(ws.a, self.W2, loc.view(-1), 1,
                                      out=ws.perm[: numel * self.W2.K].view(numel, self.W2.K))
        if fused_combine:
            if not self._combinable(B, cfg2):
                raise ValueError("fused_combine needs no norm, block_m <= 16 and the streaming decode "
                                 "kernel for the down GEMM")
            counters = ws.counters
            if counters is None or counters.numel() < M * (self.W2.N // 16):
                counters = ws.counters = ops.combine_counters(M, self.W2, x.device)
            return ops.moe_w4a16_gemm_combine(a2, self.W2, sorted_ids, eids, ntpp, topk_weights, loc, B,
                                              counters, y, out=ws.out,
                                              routed_scaling_factor=self.routed_scaling_factor, cfg=cfg2)
        ops.moe_w4a16_gemm(a2, self.W2, sorted_ids, eids, ntpp, numel, 1, B, out=y, cfg=cfg2)
        return ops.moe_combine(y, topk_weights, loc, self.norm_w, self.eps, out=ws.out,
                               routed_scaling_factor=self.routed_scaling_factor)

    __call__ = forward
