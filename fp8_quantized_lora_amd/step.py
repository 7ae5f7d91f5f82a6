"""One melded linear layer's training state and the call sequence of a step.

State (all device tensors, owned here): the E4M3 backbone codes W~ with its
fixed per-tensor scale s_w, and the adapter factors A [r x d_in] and
B [d_out x r] (B doubles as the row-wise proxy).  A step is

    fp8_quantize(X) -> melded_linear_fwd -> fp8_quantize(dY)
    -> melded_linear_bwd -> adapter_step (SGD) or adapter_step_adamw
    -> rowwise_proxy_update

With A trained and a shape whose GEMM tile grid allows it
(melded_linear_xa_fused), the forward is melded_linear_fwd_xa, which also
forms X^ A^T inside the forward FP8 product, and the backward
melded_linear_bwd_xa, which forms G^ B inside the dX product: the skinny
row-wise pass of melded_linear_bwd is not needed.  With SGD on that route, A's
pieces (the form in which the forward product takes A) are kept in a buffer:
formed at init, then left by adapter_step_pieces each time SGD moves A, and
the forward is melded_linear_fwd_xa_pieces.  When merges are periodic
(merge_every >= 2) the backbone's transpose W~^T, which the dX product reads,
is kept on that route too: formed at init by fp8_transpose, then left by
rowwise_proxy_update_t each time the proxy update rewrites W~ (the backbone
changes nowhere else in the step), and the backward is
melded_linear_bwd_xa_t, which does not transpose W~ itself.

With fp8_a=True (the pages' training setup: A frozen and held in FP8), A is
quantized once to A~ at init, the forward is melded_linear_fwd_frozen_a (Y and
U = X~ A~^T), the backward melded_linear_bwd_frozen_a (dX and dB from U), and
the proxy update's A is DQ(A~).

Every buffer and workspace is allocated once up front, so a step makes no
allocation and no host synchronisation.  This module only sequences calls
into the HIP library; it computes nothing itself.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (fp8_quantize, fp8_quantize_workspace_bytes, fp8_dequantize, melded_linear_fwd,
               melded_linear_xa_fused, melded_linear_fwd_xa, melded_linear_bwd_xa,
               melded_linear_bwd_xa_t, rowwise_proxy_update_t, fp8_transpose,
               melded_linear_fwd_xa_workspace_bytes, melded_linear_bwd_xa_workspace_bytes,
               melded_linear_bwd, melded_linear_bwd_workspace_bytes, melded_linear_fwd_frozen_a,
               melded_linear_fwd_frozen_a_workspace_bytes, melded_linear_bwd_frozen_a,
               melded_linear_bwd_frozen_a_workspace_bytes, adapter_step, adapter_step_adamw,
               adamw_state, rowwise_proxy_update, rowwise_proxy_update_workspace_bytes,
               rowwise_proxy_update_topk_rank, rowwise_proxy_update_topk_rank_workspace_bytes,
               adapter_pieces_bytes, adapter_pieces, adapter_step_pieces,
               melded_linear_fwd_xa_pieces)


class MeldedLinear:
    def __init__(self, d_out: int, d_in: int, rank: int, tokens: int, device="cuda",
                 x_dtype=torch.float32, train_a: bool = True, optimizer: str = "sgd",
                 adamw: Optional[dict] = None, fp8_a: bool = False, g_fmt: str = "e4m3",
                 topk_rank: int = 0, merge_every: int = 1):
        """optimizer "sgd" (adapter_step) or "adamw" (adapter_step_adamw, with
        hyper-parameters `adamw`: beta1, beta2, eps, weight_decay); fp8_a
        freezes A in FP8 (implies train_a=False); g_fmt is the FP8 format of the
        upstream gradient dY ("e4m3" or "e5m2"); topk_rank > 0 merges only the
        top-k rank components of the proxy (rowwise_proxy_update_topk_rank);
        merge_every: how often the caller will merge (update(merge=...)), which
        decides whether W~^T is kept (worth it from every second step on)."""
        if optimizer not in ("sgd", "adamw"):
            raise ValueError(f"optimizer must be 'sgd' or 'adamw', not {optimizer!r}")
        if fp8_a:
            train_a = False
        self.fp8_a = fp8_a
        self.g_fmt = g_fmt
        if not 0 <= topk_rank <= rank:
            raise ValueError("topk_rank must be in [0, rank]")
        self.topk_rank = topk_rank
        self.d_out, self.d_in, self.r, self.T = d_out, d_in, rank, tokens
        self.train_a = train_a
        self.optimizer = optimizer
        self.adamw = {"beta1": 0.9, "beta2": 0.999, "eps": 1e-8, "weight_decay": 0.0,
                      **(adamw or {})}

        dev = torch.device(device)
        u8, f32, i32 = torch.uint8, torch.float32, torch.int32
        self.wq = torch.empty((d_out, d_in), dtype=u8, device=dev)
        self.s_w = torch.empty(1, dtype=f32, device=dev)
        self.A = torch.empty((rank, d_in), dtype=f32, device=dev)
        self.B = torch.empty((d_out, rank), dtype=f32, device=dev)
        # per-step buffers
        self.xq = torch.empty((tokens, d_in), dtype=u8, device=dev)
        self.gq = torch.empty((tokens, d_out), dtype=u8, device=dev)
        self.s_x = torch.empty(1, dtype=f32, device=dev)
        self.s_g = torch.empty(1, dtype=f32, device=dev)
        self.y = torch.empty((tokens, d_out), dtype=f32, device=dev)
        self.dx = torch.empty((tokens, d_in), dtype=f32, device=dev)
        self.dA = torch.empty((rank, d_in), dtype=f32, device=dev) if train_a else None
        self.dB = torch.empty((d_out, rank), dtype=f32, device=dev)
        if fp8_a:                         # A~, its scale, and U = X~ A~^T of the forward
            self.aq = torch.empty((rank, d_in), dtype=u8, device=dev)
            self.s_a = torch.empty(1, dtype=f32, device=dev)
            self.u = torch.empty((tokens, rank), dtype=f32, device=dev)
        if optimizer == "adamw":          # first and second moments, zero at the start
            self.mA = torch.zeros((rank, d_in), dtype=f32, device=dev) if train_a else None
            self.vA = torch.zeros((rank, d_in), dtype=f32, device=dev) if train_a else None
            self.mB = torch.zeros((d_out, rank), dtype=f32, device=dev)
            self.vB = torch.zeros((d_out, rank), dtype=f32, device=dev)
            self.adam_state = adamw_state(dev)   # step count and beta powers, on the device
        self.sel = torch.empty(d_out, dtype=i32, device=dev)
        self.n_sel = torch.zeros(1, dtype=i32, device=dev)
        self.rho = torch.empty(d_out, dtype=f32, device=dev)
        # workspaces
        nq = max(tokens * max(d_in, d_out), d_out * d_in)
        self.ws_q = torch.empty(fp8_quantize_workspace_bytes(nq), dtype=u8, device=dev)
        # X^ A^T with the forward product, G^ B with the dX product
        self.use_xa = (not fp8_a and train_a and tokens > 0
                       and melded_linear_xa_fused(tokens, d_in, d_out, rank))
        if fp8_a:
            fw = melded_linear_fwd_frozen_a_workspace_bytes(tokens, d_in, rank)
            bw = melded_linear_bwd_frozen_a_workspace_bytes(tokens, d_in, d_out, rank)
            self.ws_fwd = torch.empty(max(1, fw), dtype=u8, device=dev)
        elif self.use_xa:
            self.xa = torch.empty((tokens, rank), dtype=f32, device=dev)
            fw = melded_linear_fwd_xa_workspace_bytes(tokens, d_in, d_out, rank)
            bw = melded_linear_bwd_xa_workspace_bytes(tokens, d_in, d_out, rank)
            self.ws_fwd = torch.empty(max(1, fw), dtype=u8, device=dev)
        # A's pieces for the fused forward, left by the SGD step that moves A
        # (A changes nowhere else in the step); formed once in init_state
        pb = adapter_pieces_bytes(rank, d_in) if self.use_xa and optimizer == "sgd" else 0
        self.keep_pieces = pb > 0
        if self.keep_pieces:
            self.a_pieces = torch.empty(pb, dtype=u8, device=dev)
        else:
            bw = melded_linear_bwd_workspace_bytes(tokens, d_in, d_out, rank)
        self.ws_bwd = torch.empty(max(1, bw), dtype=u8, device=dev)
        # W~^T for the dX product, left by the proxy update that rewrites W~
        # (not with the top-k rank proxy, whose merge leaves no transpose).
        # 4096^2: the backward's preparation without the transpose takes 4.7
        # instead of 9.8 us, the merge that writes W~^T 20.5 instead of 10.3,
        # so W~^T is kept only when merges are at most every second step
        self.keep_wt = (self.use_xa and not topk_rank and d_out % 16 == 0
                        and merge_every >= 2)
        if self.keep_wt:
            self.wqT = torch.empty((d_in, d_out), dtype=u8, device=dev)
        if topk_rank:
            self.comp_idx = torch.empty(topk_rank, dtype=i32, device=dev)
            px = rowwise_proxy_update_topk_rank_workspace_bytes(d_in, d_out, rank, topk_rank)
        else:
            px = rowwise_proxy_update_workspace_bytes(d_in, d_out, rank)
        self.ws_px = torch.empty(max(1, px), dtype=u8, device=dev)

    def init_state(self, W: torch.Tensor, A: torch.Tensor, B: torch.Tensor, stream=None):
        """W~ = E4M3(W * s_w), s_w = 448 / max|W| (the initial quantization
        error is the implicit adapter); A and B copied in."""
        fp8_quantize(W, self.wq, self.s_w, ws=self.ws_q, stream=stream)
        self.refresh_transpose(stream)
        self.B.copy_(B)
        if self.fp8_a:                    # A~ = E4M3(A * s_a); the proxy's A is DQ(A~)
            self.A.copy_(A)
            fp8_quantize(self.A, self.aq, self.s_a, ws=self.ws_q, stream=stream)
            fp8_dequantize(self.aq, self.s_a, self.A, stream=stream)
        else:
            self.A.copy_(A)
        self.refresh_pieces(stream)

    def refresh_transpose(self, stream=None):
        """Form W~^T from W~ (needed only after W~ was changed other than by
        merge)."""
        if self.keep_wt:
            fp8_transpose(self.wq, self.wqT, stream=stream)

    def refresh_pieces(self, stream=None):
        """Form A's pieces from A (needed only after A was changed other than by
        adapter_update)."""
        if self.keep_pieces:
            adapter_pieces(self.A, self.a_pieces, stream=stream)

    def forward(self, X: torch.Tensor, stream=None):
        fp8_quantize(X, self.xq, self.s_x, ws=self.ws_q, stream=stream)
        self.forward_product(stream)
        return self.y

    def forward_product(self, stream=None):
        """The forward call on the quantized activations (Y, and X^ A^T or
        X~ A~^T where the route forms it)."""
        if self.fp8_a:
            melded_linear_fwd_frozen_a(self.xq, self.s_x, self.wq, self.s_w, self.aq, self.s_a,
                                       self.y, self.u, ws=self.ws_fwd, stream=stream)
        elif self.keep_pieces:
            melded_linear_fwd_xa_pieces(self.xq, self.s_x, self.wq, self.s_w, self.a_pieces,
                                        self.r, self.y, self.xa, stream=stream)
        elif self.use_xa:
            melded_linear_fwd_xa(self.xq, self.s_x, self.wq, self.s_w, self.A, self.y, self.xa,
                                 ws=self.ws_fwd, stream=stream)
        else:
            melded_linear_fwd(self.xq, self.s_x, self.wq, self.s_w, self.y, stream=stream)

    def backward(self, dY: torch.Tensor, stream=None):
        fp8_quantize(dY, self.gq, self.s_g, ws=self.ws_q, stream=stream, fmt=self.g_fmt)
        self.backward_product(stream)
        return self.dx

    def backward_product(self, stream=None):
        """The backward call on the quantized upstream gradient (dX, dB and,
        with A trained, dA)."""
        if self.fp8_a:
            melded_linear_bwd_frozen_a(self.gq, self.s_g, self.wq, self.s_w, self.u, self.dx,
                                       self.dB, ws=self.ws_bwd, stream=stream, g_fmt=self.g_fmt)
        elif self.keep_wt:
            melded_linear_bwd_xa_t(self.gq, self.s_g, self.xq, self.s_x, self.wqT, self.s_w,
                                   self.A, self.B, self.xa, self.dx, self.dA, self.dB,
                                   ws=self.ws_bwd, stream=stream, g_fmt=self.g_fmt)
        elif self.use_xa:
            melded_linear_bwd_xa(self.gq, self.s_g, self.xq, self.s_x, self.wq, self.s_w, self.A,
                                 self.B, self.xa, self.dx, self.dA, self.dB, ws=self.ws_bwd,
                                 stream=stream, g_fmt=self.g_fmt)
        else:
            melded_linear_bwd(self.gq, self.s_g, self.xq, self.s_x, self.wq, self.s_w, self.A,
                              self.B, self.dx, self.dA, self.dB, ws=self.ws_bwd, stream=stream,
                              g_fmt=self.g_fmt)

    def adapter_update(self, lr: float, stream=None):
        if self.keep_pieces:
            adapter_step_pieces(self.A, self.B, self.dA, self.dB, lr, self.a_pieces,
                                stream=stream)
        elif self.optimizer == "sgd":
            adapter_step(self.A, self.B, self.dA, self.dB, lr, stream=stream)
        else:
            adapter_step_adamw(self.A, self.B, self.dA, self.dB, self.mA, self.vA, self.mB,
                               self.vB, self.adam_state, lr, stream=stream, **self.adamw)

    def merge(self, tau: float, k_max: int = 0, stream=None):
        if self.topk_rank:
            rowwise_proxy_update_topk_rank(self.wq, self.s_w, self.A, self.B, self.topk_rank, tau,
                                           k_max, self.sel, self.n_sel, self.comp_idx,
                                           rho=self.rho, ws=self.ws_px, stream=stream)
        elif self.keep_wt:
            rowwise_proxy_update_t(self.wq, self.wqT, self.s_w, self.A, self.B, tau, k_max,
                                   self.sel, self.n_sel, rho=self.rho, ws=self.ws_px,
                                   stream=stream)
        else:
            rowwise_proxy_update(self.wq, self.s_w, self.A, self.B, tau, k_max, self.sel,
                                 self.n_sel, rho=self.rho, ws=self.ws_px, stream=stream)

    def update(self, lr: float, tau: float, k_max: int = 0, stream=None, merge: bool = True):
        """Adapter step, then (if `merge`) the row-wise proxy update.  Between
        merges B keeps accumulating the adapter updates: B is the proxy, merged
        into W~ periodically."""
        self.adapter_update(lr, stream)
        if merge:
            self.merge(tau, k_max, stream)

    def step(self, X: torch.Tensor, dY: torch.Tensor, lr: float = 1e-3, tau: float = 0.5,
             k_max: int = 0, stream=None, merge_every: int = 1):
        """One training step; the proxy is merged into W~ on every
        `merge_every`-th step (counted by this layer)."""
        if merge_every < 1:
            raise ValueError("merge_every must be >= 1")
        self.n_steps = getattr(self, "n_steps", 0) + 1
        self.forward(X, stream)
        self.backward(dY, stream)
        self.update(lr, tau, k_max, stream, merge=self.n_steps % merge_every == 0)
