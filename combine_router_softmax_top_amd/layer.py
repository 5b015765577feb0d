"""Device buffers of one MoE layer call and stage-by-stage calls of the C ABI.

Plumbing only: it allocates torch device memory for inputs, outputs and
workspaces and calls the binding; every step runs in the HIP library.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import binding as B
from .workloads import MoEConfig


class MoELayer:
    WEIGHTS = ("w_router", "bias", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")

    def __init__(self, cfg: MoEConfig, host_inputs: dict, device: str = "cuda",
                 share_weights: Optional["MoELayer"] = None):
        """share_weights: another layer of the same shape except the token
        count, whose device weights this one uses instead of copies."""
        self.cfg = cfg
        self.cs = B.config_struct(cfg)
        dev = torch.device(device)
        self.device = dev
        T, d, E, K = cfg.num_tokens, cfg.hidden, cfg.num_experts, cfg.top_k
        S, n_loc, dt = cfg.num_shared, cfg.num_local, cfg.torch_dtype

        def to_dev(t):
            return None if t is None else t.to(dev, non_blocking=False).contiguous()

        self.x = to_dev(host_inputs["x"])
        if share_weights is not None:
            o = share_weights.cfg
            keys = ("hidden", "num_experts", "intermediate", "expert_begin", "expert_end",
                    "num_shared", "dtype", "router_init", "zipf_s", "packed_weights")
            if any(getattr(o, k) != getattr(cfg, k) for k in keys):
                raise ValueError("share_weights: the layers' weights differ")
            for name in self.WEIGHTS:
                setattr(self, name, getattr(share_weights, name))
        else:
            for name in self.WEIGHTS:
                setattr(self, name, to_dev(host_inputs.get(name)))
        if cfg.packed_weights and share_weights is None:
            # the bf16 stacks rearranged once, like an offline conversion
            for name in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
                w = getattr(self, name)
                if w is not None:
                    packed = torch.empty_like(w)
                    B.moe_pack_weights(w, packed)
                    setattr(self, name, packed)
            torch.cuda.synchronize(dev)

        self.topk_ids = torch.empty(T, K, dtype=torch.int32, device=dev)
        self.topk_weights = torch.empty(T, K, dtype=torch.float32, device=dev)
        self.logits = torch.empty(T, E, dtype=torch.float32, device=dev)
        self.counts = torch.empty(E, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(n_loc + 1, dtype=torch.int32, device=dev)
        self.x_sorted = torch.empty(T * K, d, dtype=dt, device=dev)
        self.src_index = torch.empty(T * K, dtype=torch.int32, device=dev)
        self.row_of = torch.empty(T * K, dtype=torch.int32, device=dev)
        self.y_sorted = torch.empty(T * K, d, dtype=dt, device=dev)
        self.y_shared = torch.empty(S, T, d, dtype=dt, device=dev) if S > 0 else None
        self.out = torch.empty(T, d, dtype=dt, device=dev)
        self.ws_route = B.alloc_workspace(self.cs, B.MOE_WS_ROUTE, dev)
        self.ws_dispatch = B.alloc_workspace(self.cs, B.MOE_WS_DISPATCH, dev)
        self.ws_mlp = B.alloc_workspace(self.cs, B.MOE_WS_EXPERT_MLP, dev)
        self._ws_forward: Optional[torch.Tensor] = None
        self._ws_dbo: Optional[torch.Tensor] = None
        self.mx: Optional[dict] = None  # MX-FP8 gate / up weights (quantize_weights)

    # ---- block-scaled (MX-FP8) path ------------------------------------------
    def quantize_weights(self, down: bool = False) -> dict:
        """MX-FP8 encodings of the gate and up stacks (and, with down=True, of
        the down stack), routed and shared, in the MFMA scale layout, done once
        like an offline weight conversion."""
        c = self.cfg
        n_loc, I, d, S = c.num_local, c.intermediate, c.hidden, c.num_shared
        mx = {}
        mats = [("wq_gate", self.w_gate, I, d), ("wq_up", self.w_up, I, d)]
        if down:
            mats.append(("wq_down", self.w_down, d, I))
        if S > 0:
            mats += [("wsq_gate", self.ws_gate, I, d), ("wsq_up", self.ws_up, I, d)]
            if down:
                mats.append(("wsq_down", self.ws_down, d, I))
        for name, w, rows, cols in mats:
            n = w.shape[0]
            codes = torch.empty(n, rows, cols, dtype=torch.uint8, device=self.device)
            scales = torch.empty(n * rows * cols // 32, dtype=torch.uint8, device=self.device)
            B.moe_quantize_mxfp8(w.view(n * rows, cols), codes.view(n * rows, cols), scales,
                                 B.MOE_MX_MFMA)
            mx[name], mx[name + "_scales"] = codes, scales
        self.mx = mx
        return mx

    def tensors_mxfp8(self, out: Optional[torch.Tensor] = None) -> dict:
        """Tensors of the block-scaled layer: the down projection in MX-FP8 when
        quantize_weights(down=True) was called, else in bf16."""
        if self.mx is None:
            self.quantize_weights()
        t = dict(x=self.x, w_router=self.w_router, bias=self.bias,
                 out=self.out if out is None else out, topk_ids=self.topk_ids,
                 topk_weights=self.topk_weights, **self.mx)
        if "wq_down" not in self.mx:
            t["w_down"] = self.w_down
            if self.cfg.num_shared > 0:
                t["ws_down"] = self.ws_down
        return t

    def forward_mxfp8(self, stream=None, out: Optional[torch.Tensor] = None):
        if self._ws_forward is None:
            self._ws_forward = B.alloc_workspace(self.cs, B.MOE_WS_FORWARD, self.device)
        B.moe_forward_mxfp8(self.cs, self.tensors_mxfp8(out), self._ws_forward, stream)

    # ---- stages -------------------------------------------------------------
    def route(self, stream=None, with_logits: bool = True):
        B.moe_route(self.cs, self.x, self.w_router, self.bias, self.topk_ids, self.topk_weights,
                    self.logits if with_logits else None, self.ws_route, stream)

    def dispatch(self, stream=None, topk_ids: Optional[torch.Tensor] = None):
        B.moe_dispatch(self.cs, self.x, self.topk_ids if topk_ids is None else topk_ids,
                       self.counts, self.offsets, self.x_sorted, self.src_index, self.row_of,
                       self.ws_dispatch, stream)

    def expert_mlp(self, stream=None):
        B.moe_expert_mlp(self.cs, self.x_sorted, self.offsets, self.w_gate, self.w_up,
                         self.w_down, self.y_sorted, self.x if self.cfg.num_shared else None,
                         self.ws_gate, self.ws_up, self.ws_down, self.y_shared, self.ws_mlp,
                         stream)

    def combine(self, stream=None, out: Optional[torch.Tensor] = None):
        B.moe_combine(self.cs, self.y_sorted, self.row_of, self.topk_weights, self.y_shared,
                      self.out if out is None else out, stream)

    def n_invalid(self) -> int:
        return int(self.ws_dispatch[:4].view(torch.int32).item())

    # ---- whole layer --------------------------------------------------------
    def tensors(self, out: Optional[torch.Tensor] = None) -> dict:
        return dict(x=self.x, w_router=self.w_router, bias=self.bias, w_gate=self.w_gate,
                    w_up=self.w_up, w_down=self.w_down, ws_gate=self.ws_gate, ws_up=self.ws_up,
                    ws_down=self.ws_down, out=self.out if out is None else out,
                    topk_ids=self.topk_ids, topk_weights=self.topk_weights)

    def forward(self, stream=None, out: Optional[torch.Tensor] = None):
        if self._ws_forward is None:
            self._ws_forward = B.alloc_workspace(self.cs, B.MOE_WS_FORWARD, self.device)
        B.moe_forward(self.cs, self.tensors(out), self._ws_forward, stream)

    def forward_dbo(self, compute=None, comm=None, min_tokens_to_split: int = 0,
                    out: Optional[torch.Tensor] = None, split: Optional[int] = None):
        """moe_forward_dbo (midpoint cut), or moe_forward_dbo_at with split given."""
        if self._ws_dbo is None:
            self._ws_dbo = B.alloc_workspace(self.cs, B.MOE_WS_FORWARD_DBO, self.device)
        if split is None:
            B.moe_forward_dbo(self.cs, self.tensors(out), self._ws_dbo, min_tokens_to_split,
                              compute, comm)
        else:
            B.moe_forward_dbo_at(self.cs, self.tensors(out), self._ws_dbo, split, compute, comm)

    def capture_forward(self, out: Optional[torch.Tensor] = None, dbo: bool = False,
                        min_tokens_to_split: int = 0) -> B.Graph:
        """The whole layer (moe_forward, or moe_forward_dbo with dbo=True) captured
        as a HIP graph over this layer's buffers; replay with .launch(stream)."""
        if dbo:
            if self._ws_dbo is None:
                self._ws_dbo = B.alloc_workspace(self.cs, B.MOE_WS_FORWARD_DBO, self.device)
            ws = self._ws_dbo
        else:
            if self._ws_forward is None:
                self._ws_forward = B.alloc_workspace(self.cs, B.MOE_WS_FORWARD, self.device)
            ws = self._ws_forward
        return B.moe_graph_capture_forward(self.cs, self.tensors(out), ws, dbo=dbo,
                                           min_tokens_to_split=min_tokens_to_split)

    def capture_forward_mxfp8(self, out: Optional[torch.Tensor] = None) -> B.Graph:
        """The block-scaled layer (moe_forward_mxfp8) captured as a HIP graph."""
        if self._ws_forward is None:
            self._ws_forward = B.alloc_workspace(self.cs, B.MOE_WS_FORWARD, self.device)
        return B.moe_graph_capture_forward_mxfp8(self.cs, self.tensors_mxfp8(out),
                                                 self._ws_forward)

    def n_rows(self) -> int:
        return int(self.offsets[-1].item())
