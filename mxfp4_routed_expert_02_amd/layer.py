"""A routed-expert layer object: owns the workspace and output buffers for a
maximum token count and issues the C-ABI calls on the current stream: for one
token the whole layer in one call (moe_decode_layer_mxfp4); for several,
route and group, then the expert FFN with the combine
(moe_expert_ffn_combine_mxfp4).
Reusing one object across stacked layers reuses its buffers (the buffers of
one layer template serve every layer)."""
from __future__ import annotations

from typing import Optional

import torch

from . import _binding as B


class RoutedExpertLayer:
    def __init__(self, E: int, H: int, I: int, k: int, max_tokens: int, device="cuda"):
        self.E, self.H, self.I, self.k, self.max_tokens = E, H, I, k, max_tokens
        self.device = torch.device(device)
        ws = B.workspace_bytes(max_tokens, k, E, H, I)
        if ws == 0:
            raise ValueError("shape outside the library's supported ranges")
        R = max_tokens * k
        dev = self.device
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
        self.ids = torch.empty((max_tokens, k), dtype=torch.int32, device=dev)
        self.weights = torch.empty((max_tokens, k), dtype=torch.float32, device=dev)
        self.grp = B.Grouping(torch.empty(E + 1, dtype=torch.int32, device=dev),
                              torch.empty(R, dtype=torch.int32, device=dev),
                              torch.empty(R, dtype=torch.int32, device=dev),
                              torch.empty(E + 1, dtype=torch.int32, device=dev))
        self.y_rows = torch.empty((R, H), dtype=torch.float32, device=dev)
        self.out = torch.empty((max_tokens, H), dtype=torch.float32, device=dev)

    def _views(self, T: int):
        R = T * self.k
        grp = B.Grouping(self.grp.expert_offsets, self.grp.sorted_rows[:R], self.grp.row_pos[:R], self.grp.active)
        return self.ids[:T], self.weights[:T], grp, self.y_rows[:R], self.out[:T]

    def route(self, logits: torch.Tensor):
        T = logits.shape[0]
        ids, w, grp, _, _ = self._views(T)
        B.route_topk(logits, self.k, ids, w)
        B.group_rows(ids, self.E, self.workspace, grp)
        return ids, w, grp

    def __call__(self, x: torch.Tensor, logits: torch.Tensor, pool: B.ExpertPool,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """x [T, H] bf16, logits [T, E] fp32 -> out [T, H] fp32."""
        T = x.shape[0]
        if T > self.max_tokens:
            raise ValueError("more tokens than the layer was sized for")
        ids, w, grp, y_rows, o = self._views(T)
        o = o if out is None else out
        if T == 1:  # the whole layer in one call (two launches at the decode shape)
            return B.decode_layer_mxfp4(logits, x, self.k, pool, ids, w, grp, self.workspace, y_rows, o)
        self._route_group(logits, ids, w, grp)
        return B.expert_ffn_combine_mxfp4(x, self.k, pool, grp, w, self.workspace, y_rows, o)

    def _route_group(self, logits, ids, w, grp):
        if logits.shape[0] == 1:  # one token: top-k and grouping in one launch
            B.route_group_one(logits, self.k, ids, w, grp)
        else:
            B.route_topk(logits, self.k, ids, w)
            B.group_rows(ids, self.E, self.workspace, grp)

    def step(self, x: torch.Tensor, logits: torch.Tensor, pool: B.ExpertPool, out: torch.Tensor,
             x_next: torch.Tensor, eps: float = 1e-6) -> torch.Tensor:
        """One layer of a stack: out [T, H] fp32 as __call__ gives it, and
        x_next [T, H] bf16 = its RMS rescale, the next layer's input (the
        combine and the rescale in one launch)."""
        T = x.shape[0]
        if T > self.max_tokens:
            raise ValueError("more tokens than the layer was sized for")
        ids, w, grp, y_rows, _ = self._views(T)
        if T == 1:  # the layer in one call, then the rescale
            B.decode_layer_mxfp4(logits, x, self.k, pool, ids, w, grp, self.workspace, y_rows, out)
            return B.rms_rescale_bf16(out, eps, x_next)
        self._route_group(logits, ids, w, grp)
        B.expert_ffn_mxfp4(x, self.k, pool, grp, self.workspace, y_rows)
        return B.combine_rms_bf16(y_rows, w, grp.row_pos, out, x_next, eps)

    def step_rms(self, y_prev: torch.Tensor, logits: torch.Tensor, pool: B.ExpertPool, out: torch.Tensor,
                 x_used: torch.Tensor, eps: float = 1e-6) -> torch.Tensor:
        """One stacked layer fed by the previous layer's output: x_used [1, H]
        bf16 = RMS rescale of y_prev [1, H] fp32, then the layer on it into
        out [1, H] fp32 (out may be y_prev's own buffer).  One token only; at
        the decode shape the rescale runs inside the gate/up launch."""
        if y_prev.shape[0] != 1:
            raise ValueError("step_rms takes one token")
        ids, w, grp, y_rows, _ = self._views(1)
        return B.decode_layer_rms_mxfp4(logits, y_prev, eps, x_used, self.k, pool, ids, w, grp, self.workspace,
                                        y_rows, out)
