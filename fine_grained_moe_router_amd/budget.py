"""Algorithmic byte counts of the decode step (host-side arithmetic, no GPU).

A batch-1 decode step is a chain of GEMVs at about one FLOP per weight byte, so
its time is set by the weight bytes it must stream (page 'LLM decoding',
us-homepage.pages.dev/blog/llm-decoding, sections "First principles:
compute-bound or memory-bound?" and "Where the 7.36 GB goes"). These helpers count
those bytes for the shapes used here: each weight byte the step needs is counted
once per step, whatever the number of tokens M sharing it; work the sparse step
avoids (unselected experts) is not counted.
"""
from __future__ import annotations

HBM_PEAK_BYTES_PER_S = 8.0e12  # MI355X HBM3E, vendor figure


def expert_bytes(hidden: int, width: int, weight_bytes: int = 1, scales: bool = True) -> int:
    """gate [F][H] + up [F][H] + down [H][F] weights, plus fp32 per-row scales."""
    b = 3 * width * hidden * weight_bytes
    if scales:
        b += (2 * width + hidden) * 4
    return b


def router_bytes(hidden: int, experts: int, bias: bool = False, router_dtype: str = "bf16") -> int:
    """bf16 [H][E], or FP8 codes [H][E] with one fp32 scale per expert; the bias if any."""
    w = hidden * experts * 2 if router_dtype == "bf16" else hidden * experts + experts * 4
    return w + (experts * 4 if bias else 0)


def lm_head_bytes(vocab: int, hidden: int) -> int:
    """FP8 codes plus one fp32 scale per row."""
    return vocab * hidden + vocab * 4


def layer_bytes(shape, unique_routed: int, M: int, expert_dtype: str = "fp8",
                bias: bool = False, norm: bool = False, router_dtype: str = "bf16") -> int:
    """One MoE layer: the router, each expert in the union once, the shared expert,
    and the bf16 activations (input read, output written; with the residual norm
    also the residual, the noise and the gain)."""
    wb = 1 if expert_dtype == "fp8" else 2
    sc = expert_dtype == "fp8"
    H = shape.hidden
    b = router_bytes(H, shape.experts, bias, router_dtype)
    b += unique_routed * expert_bytes(H, shape.width, wb, sc)
    if shape.shared_width:
        b += expert_bytes(H, shape.shared_width, wb, sc)
    b += 2 * M * H * 2
    if norm:
        b += 3 * M * H * 2 + H * 2 + M * H * 2
    return b


def step_bytes(shape, unique_routed_per_layer, M: int, expert_dtype: str = "fp8",
               bias: bool = False, lm_dtype: str = "fp8", router_dtype: str = "bf16") -> int:
    """Whole stacked step: every layer (with its residual norm), the final norm, the
    lm_head (FP8 codes and row scales, or bf16), and the argmax / acceptance outputs
    (negligible, counted as 16 B/token)."""
    b = 0
    for u in unique_routed_per_layer:
        b += layer_bytes(shape, int(u), M, expert_dtype, bias, norm=True, router_dtype=router_dtype)
    H = shape.hidden
    b += 3 * M * H * 2 + H * 2            # final residual add + norm
    b += lm_head_bytes(shape.vocab, H) if lm_dtype == "fp8" else 2 * shape.vocab * H
    b += 16 * M
    return b


def expected_unique(experts: int, top_k: int, M: int) -> float:
    """E|union of M uniform top-K draws| = E (1 - (1 - K/E)^M)."""
    return experts * (1.0 - (1.0 - top_k / experts) ** M)


def bf16_token_budget(hidden, experts_per_token, width, layers, vocab, shared_width,
                      router_experts, attention_params):
    """The BF16 per-token weight budget, matrix family by matrix family (2 B/param):
    routed experts (3 matrices each), attention (given as a parameter count), tied
    lm_head, shared MLP (3 matrices), router. Returns params and bytes per family."""
    p = {
        "experts": experts_per_token * 3 * hidden * width * layers,
        "attention": attention_params,
        "lm_head": vocab * hidden,
        "dense_mlp": 3 * hidden * shared_width * layers,
        "router": hidden * router_experts * layers,
    }
    b = {k: 2 * v for k, v in p.items()}
    b["total"] = sum(b.values())
    return p, b
