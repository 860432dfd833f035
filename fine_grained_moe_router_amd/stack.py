"""The stacked decode step: L MoE layers with a residual RMSNorm before each, the
final norm, the tied lm_head + argmax and greedy acceptance, driven through the C
ABI (argument marshalling only; every step runs in libmoedecode's kernels).

    h_0 = x
    for l: (h, u_l) = add_rmsnorm(h, noise_l, y_{l-1}; g_l);  y_l = moe_decode_layer(u_l)
    (h, x_f) = add_rmsnorm(h, y_{L-1}; g_L)
    tok = lm_head_argmax(x_f);  (n, out) = spec_accept(drafts, tok)

Attention is not part of this step; the stacked workload adds noise in its place.
All buffers are allocated once here; a step allocates nothing and can be captured
in a HIP graph.
"""
from __future__ import annotations

import torch

from . import native


class DecodeStack:
    def __init__(self, shape, layers, gains, lm_w, lm_s, max_M: int, expert_dtype: str = "fp8",
                 eps: float = 1e-6, device="cuda"):
        self.shape = shape
        self.L = len(layers)
        self.max_M = max_M
        self.eps = eps
        self.layers = layers                      # keep the tensors alive
        self.desc = native.layer_desc(shape, expert_dtype, layers[0].get("router_dtype", "bf16"))
        self.lw = [native.layer_weights(w) for w in layers]
        self.gains = gains
        self.lm_w, self.lm_s = lm_w, lm_s
        H, K = shape.hidden, shape.top_k
        self.ws_bytes = native.moe_decode_layer_workspace(self.desc, max_M)
        if self.ws_bytes == 0:
            raise ValueError("unsupported layer shape for the decode library")
        self.ws = native.workspace(self.ws_bytes, device)
        self.lm_ws_bytes = native.lm_head_argmax_workspace(max_M, H, shape.vocab)
        self.lm_ws = native.workspace(self.lm_ws_bytes, device)
        z = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt, device=device)
        self.h = z(max_M, H)
        self.u = z(self.L, max_M, H)
        self.y = z(self.L, max_M, H)
        self.x_final = z(max_M, H)
        self.topk_idx = z(self.L, max_M, K, dt=torch.int32)
        self.topk_w = z(self.L, max_M, K, dt=torch.float32)
        self.tok = z(max_M, dt=torch.int32)
        self.max_logit = z(max_M, dt=torch.float32)
        self.accepted = z(4, dt=torch.int32)
        self.out_tokens = z(max_M, dt=torch.int32)

    def step(self, x, noise, drafts, M: int, stream=None):
        """One decode step for M tokens. x bf16 [M][H]; noise bf16 [L][M][H];
        drafts int32 [M-1] (ignored when M == 1)."""
        sh, H = self.shape, self.shape.hidden
        h = self.h[:M]
        for l in range(self.L):
            native.moe_add_rmsnorm(M, H, x if l == 0 else h, noise[l], None if l == 0 else self.y[l - 1, :M],
                                   self.gains[l], self.eps, h, self.u[l, :M], stream)
            native.moe_decode_layer(self.desc, self.lw[l], M, self.u[l, :M], self.y[l, :M],
                                    self.topk_idx[l, :M], self.topk_w[l, :M], self.ws, self.ws_bytes,
                                    stream)
        native.moe_add_rmsnorm(M, H, h, self.y[self.L - 1, :M], None, self.gains[self.L], self.eps, h,
                               self.x_final[:M], stream)
        native.lm_head_argmax(M, H, sh.vocab, self.x_final[:M], self.lm_w, self.lm_s, self.tok[:M],
                              self.max_logit[:M], self.lm_ws, self.lm_ws_bytes, stream)
        native.spec_accept(M - 1, drafts if M > 1 else None, self.tok[:M], self.accepted,
                           self.out_tokens[:M], stream)


class FusedDecodeStep:
    """The same step as DecodeStack, run by the library's single-launch entry point
    moe_decode_step (one persistent kernel per step)."""

    def __init__(self, shape, layers, gains, lm_w, lm_s, max_M: int, eps: float = 1e-6,
                 spin_limit: int = 0, device="cuda", cooperative: bool = False):
        self.shape = shape
        self.L = len(layers)
        self.max_M = max_M
        self.layers = layers
        self.gains, self.lm_w, self.lm_s = gains, lm_w, lm_s
        expert_dtype = layers[0].get("expert_dtype", "fp8")
        self.lm_bf16 = lm_w.dtype == torch.bfloat16      # the BF16 rung: [V][H] bf16, no scales
        self.desc = native.step_desc(shape.with_(layers=self.L), max_M, eps, spin_limit, expert_dtype,
                                     cooperative, self.lm_bf16, layers[0].get("router_dtype", "bf16"))
        self.ws_bytes = native.moe_decode_step_workspace(self.desc)
        if self.ws_bytes == 0:
            raise ValueError("unsupported shape for the fused decode step")
        self.ws = native.workspace(self.ws_bytes, device)
        native.moe_decode_step_prepare(self.desc, [native.layer_weights(w) for w in layers], self.ws,
                                       self.ws_bytes)
        H, K, L = shape.hidden, shape.top_k, self.L
        z = lambda n, dt: torch.zeros(n, dtype=dt, device=device)
        self._y = z(L * max_M * H, torch.bfloat16)
        self._idx = z(L * max_M * K, torch.int32)
        self._w = z(L * max_M * K, torch.float32)
        self.x_final = torch.zeros(max_M, H, dtype=torch.bfloat16, device=device)
        self.tok = z(max_M, torch.int32)
        self.max_logit = z(max_M, torch.float32)
        self.accepted = z(4, torch.int32)
        self.out_tokens = z(max_M, torch.int32)
        self.M = max_M

    def y(self, M=None):
        M = M or self.M
        return self._y[: self.L * M * self.shape.hidden].view(self.L, M, self.shape.hidden)

    def topk_idx(self, M=None):
        M = M or self.M
        return self._idx[: self.L * M * self.shape.top_k].view(self.L, M, self.shape.top_k)

    def topk_w(self, M=None):
        M = M or self.M
        return self._w[: self.L * M * self.shape.top_k].view(self.L, M, self.shape.top_k)

    def step(self, x, noise, drafts, M: int, stream=None, outputs: bool = True):
        """One step for M tokens; outputs=False skips the per-layer diagnostic outputs."""
        self.M = M
        native.moe_decode_step(self.desc, M, self.gains, self.lm_w, self.lm_s, x, noise,
                               drafts if M > 1 else None, self.tok[:M], self.max_logit[:M],
                               self.accepted, self.out_tokens[:M],
                               self._y if outputs else None, self._idx if outputs else None,
                               self._w if outputs else None, self.x_final if outputs else None,
                               self.ws, self.ws_bytes, stream)

    def status(self) -> int:
        return native.moe_decode_step_status(self.desc, self.ws)
