"""Seeded synthetic weights and inputs for the batch-1 fine-grained MoE decode step.

This module is the only code that both the CPU oracle tests and the GPU path use.
It draws random numbers with seeded torch generators and stores them in the
formats the decode step consumes:

* bf16 tensors (router weights, hidden vectors, RMSNorm gains, noise),
* OCP E4M3FN code bytes with one fp32 scale per output row (expert matrices and the
  tied lm_head), made the way a load-time FP8 weight-only quantiser makes them:
  scale = row absmax / 448, code = round-to-nearest-even E4M3FN of (w / scale),
  done by torch's own float8 conversion.

It holds none of the decode step's arithmetic (no routing, no GEMV, no argmax,
no acceptance). Random draws are keyed by (seed, tag, kind, layer, index) through
SHA-256, so any block can be regenerated on its own. The same key on a different
device gives different numbers (torch's CPU and GPU generators differ); a test
generates on one device and copies to the other.

Shapes follow the Gemma-4-26B-A4B description on the page 'LLM decoding'
(us-homepage.pages.dev/blog/llm-decoding), section "The exact architecture, and
why it rules out 4-bit": hidden 2816, 128 experts, top-8 plus one shared expert,
expert width 704, 30 layers, tied vocabulary 262,144.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np
import torch

FP8_MAX = 448.0  # largest finite OCP E4M3FN magnitude


@dataclasses.dataclass(frozen=True)
class Shape:
    hidden: int
    experts: int
    top_k: int
    width: int          # routed expert FFN width
    shared_width: int   # shared expert FFN width (0: no shared expert)
    vocab: int
    layers: int = 1

    def with_(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


# Gemma-4-26B-A4B-shaped layer (shared expert at the routed width; the page's
# 2112-wide dense MLP is available through with_(shared_width=2112)).
GEMMA4_26B_A4B = Shape(hidden=2816, experts=128, top_k=8, width=704,
                       shared_width=704, vocab=262144, layers=30)
# Tiny parity shape: hidden 256, 16 experts top-2 plus shared, width 64, vocab 4096.
TINY = Shape(hidden=256, experts=16, top_k=2, width=64, shared_width=64,
             vocab=4096, layers=1)

ROUTER_STD = 0.05
EXPERT_STD = 0.02
LM_HEAD_STD = 0.02
NOISE_STD = 0.1
GAIN_MEAN, GAIN_STD = 1.0, 0.1


def seed_of(*key) -> int:
    """A 63-bit seed from an arbitrary tuple key (stable across runs and hosts)."""
    digest = hashlib.sha256(repr(key).encode()).digest()
    return int.from_bytes(digest[:8], "little") & ((1 << 63) - 1)


def _gen(device, *key) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*key))
    return g


def normal(shape, std, device, *key, mean=0.0) -> torch.Tensor:
    g = _gen(device, *key)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t


def quantize_rows_fp8(w: torch.Tensor):
    """Per-output-row FP8 (E4M3FN) codes and fp32 scales of a float32 matrix.

    Rows are the last-but-one axis: w[..., row, col]. Returns (codes uint8, scales fp32).
    An all-zero row gets scale 0 and code 0.
    """
    amax = w.abs().amax(dim=-1)
    scale = amax / FP8_MAX
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    q = (w / safe.unsqueeze(-1)).clamp_(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale.contiguous()


def _fp8_matrix(shape, std, device, *key):
    """Draw N(0, std) and quantise per row; done in slices to bound temporaries."""
    lead = shape[0]
    codes = torch.empty(shape, dtype=torch.uint8, device=device)
    scales = torch.empty(shape[:-1], dtype=torch.float32, device=device)
    per = max(1, (1 << 27) // max(1, int(np.prod(shape[1:]))))
    for i0 in range(0, lead, per):
        i1 = min(lead, i0 + per)
        w = normal((i1 - i0,) + tuple(shape[1:]), std, device, *key, i0)
        codes[i0:i1], scales[i0:i1] = quantize_rows_fp8(w)
        del w
    return codes, scales


def router_weights(shape: Shape, layer: int = 0, device="cpu", seed: int = 0, tag: str = "moe",
                   router_dtype: str = "bf16") -> dict:
    """The router of layer_weights() alone: router_w (bf16 [H][E], or FP8 codes [H][E] quantised
    per expert from the same draws), router_s (fp32 [E] or None) and router_dtype."""
    H, E = shape.hidden, shape.experts
    rw = normal((H, E), ROUTER_STD, device, seed, tag, layer, "router")
    if router_dtype == "fp8":
        codes, rs = quantize_rows_fp8(rw.t().contiguous())
        return {"router_w": codes.t().contiguous(), "router_s": rs, "router_dtype": "fp8"}
    if router_dtype == "bf16":
        return {"router_w": rw.to(torch.bfloat16), "router_s": None, "router_dtype": "bf16"}
    raise ValueError(router_dtype)


def layer_weights(shape: Shape, layer: int = 0, device="cpu", seed: int = 0,
                  tag: str = "moe", expert_dtype: str = "fp8",
                  router_bias: Optional[torch.Tensor] = None, router_dtype: str = "bf16") -> dict:
    """Weights of one MoE layer in the boundary's logical row-major layout.

    router_w  bf16 [H][E]            N(0, 0.05); with router_dtype="fp8" the same draws as
              FP8 codes [H][E] quantised per expert (column), scales router_s fp32 [E]
    router_b  fp32 [E] or None
    gate_w/up_w  [E][D][H], down_w [E][H][D]: uint8 FP8 codes (expert_dtype="fp8",
              with fp32 per-row scales gate_s/up_s [E][D], down_s [E][H]) or bf16
              (expert_dtype="bf16", scales None); values N(0, 0.02) before quantisation.
    sh_*      the shared expert: [Ds][H], [Ds][H], [H][Ds] (None when Ds == 0).
    """
    H, E, D, Ds = shape.hidden, shape.experts, shape.width, shape.shared_width
    k = (seed, tag, layer)
    out = {"router_b": None if router_bias is None else router_bias.to(device=device, dtype=torch.float32)}
    out.update(router_weights(shape, layer, device, seed, tag, router_dtype))

    def mat(shp, name):
        if expert_dtype == "fp8":
            return _fp8_matrix(shp, EXPERT_STD, device, *k, name)
        if expert_dtype == "bf16":
            w = torch.empty(shp, dtype=torch.bfloat16, device=device)
            for i in range(shp[0]):
                w[i] = normal(tuple(shp[1:]), EXPERT_STD, device, *k, name, i).to(torch.bfloat16)
            return w, None
        raise ValueError(expert_dtype)

    out["gate_w"], out["gate_s"] = mat((E, D, H), "gate")
    out["up_w"], out["up_s"] = mat((E, D, H), "up")
    out["down_w"], out["down_s"] = mat((E, H, D), "down")
    if Ds > 0:
        for name, shp in (("gate", (Ds, H)), ("up", (Ds, H)), ("down", (H, Ds))):
            w, s = mat((1,) + shp, "shared_" + name)
            out["sh_%s_w" % name] = w[0]
            out["sh_%s_s" % name] = None if s is None else s[0]
    else:
        for name in ("gate", "up", "down"):
            out["sh_%s_w" % name] = None
            out["sh_%s_s" % name] = None
    out["expert_dtype"] = expert_dtype
    return out


def lm_head(shape: Shape, device="cpu", seed: int = 0, tag: str = "lm_head"):
    """Tied lm_head [V][H]: FP8 codes from N(0, 0.02) with per-row fp32 scales."""
    return _fp8_matrix((shape.vocab, shape.hidden), LM_HEAD_STD, device, seed, tag)


def lm_head_bf16(shape: Shape, device="cpu", seed: int = 0, tag: str = "lm_head") -> torch.Tensor:
    """Tied lm_head [V][H] in bf16: the same N(0, 0.02) draws as lm_head(), rounded once to
    bf16 instead of quantised (the precision ladder's BF16 rung)."""
    V, H = shape.vocab, shape.hidden
    out = torch.empty((V, H), dtype=torch.bfloat16, device=device)
    per = max(1, (1 << 27) // H)
    for i0 in range(0, V, per):
        i1 = min(V, i0 + per)
        out[i0:i1] = normal((i1 - i0, H), LM_HEAD_STD, device, seed, tag, i0).to(torch.bfloat16)
    return out


@dataclasses.dataclass(frozen=True)
class DraftShape:
    """The MTP drafter head (page 'LLM decoding', "The one-line shape bug that disabled the
    model's own drafter": a 5632 = 2 x 2816 -> 1024 pre_projection and a 1024-wide own
    embedding table; "Lever 2": a 430M head). The body's depth and width are a reading: 12
    GELU-gated MLP blocks of width 4096, so the head holds about 430M parameters."""
    hidden: int = 2816      # the target's width (embedding and hidden state)
    width: int = 1024       # the head's width
    ffn: int = 4096         # the blocks' inner width
    blocks: int = 12
    vocab: int = 262144

    def params(self) -> int:
        D, F, H, V = self.width, self.ffn, self.hidden, self.vocab
        return D * 2 * H + self.blocks * 3 * D * F + V * D + H * D


MTP_HEAD = DraftShape()
TINY_HEAD = DraftShape(hidden=256, width=256, ffn=512, blocks=2, vocab=1024)


def draft_head(shape: DraftShape, device="cpu", seed: int = 0, tag: str = "mtp") -> dict:
    """The drafter head's weights: FP8 codes with per-row fp32 scales (N(0, 0.02) draws
    quantised like the experts) and bf16 RMSNorm gains N(1, 0.1) ([blocks + 1][width], the
    last the final norm's). Block matrices are stacked: gate_w, up_w [blocks][ffn][width],
    down_w [blocks][width][ffn]."""
    D, F, H, V, B = shape.width, shape.ffn, shape.hidden, shape.vocab, shape.blocks
    out = {}
    out["pre_w"], out["pre_s"] = _fp8_matrix((D, 2 * H), EXPERT_STD, device, seed, tag, "pre")
    out["gate_w"], out["gate_s"] = _fp8_matrix((B, F, D), EXPERT_STD, device, seed, tag, "gate")
    out["up_w"], out["up_s"] = _fp8_matrix((B, F, D), EXPERT_STD, device, seed, tag, "up")
    out["down_w"], out["down_s"] = _fp8_matrix((B, D, F), EXPERT_STD, device, seed, tag, "down")
    out["table_w"], out["table_s"] = _fp8_matrix((V, D), LM_HEAD_STD, device, seed, tag, "table")
    out["post_w"], out["post_s"] = _fp8_matrix((H, D), EXPERT_STD, device, seed, tag, "post")
    out["gains"] = normal((B + 1, D), GAIN_STD, device, seed, tag, "gain", mean=GAIN_MEAN).to(torch.bfloat16)
    return out


def draft_head_to_host(w: dict, shape: DraftShape) -> dict:
    """The layout oracle.draft_step takes: numpy arrays, blocks as a list of dicts."""
    h = {k: (bytes8(v) if v.dtype == torch.uint8 else (bits16(v) if v.dtype == torch.bfloat16 else f32(v)))
         for k, v in w.items()}
    blocks = [{"gain": h["gains"][b], "gate_w": h["gate_w"][b], "gate_s": h["gate_s"][b], "up_w": h["up_w"][b],
               "up_s": h["up_s"][b], "down_w": h["down_w"][b], "down_s": h["down_s"][b]}
              for b in range(shape.blocks)]
    return {"pre_w": h["pre_w"], "pre_s": h["pre_s"], "blocks": blocks, "final_gain": h["gains"][shape.blocks],
            "table_w": h["table_w"], "table_s": h["table_s"], "post_w": h["post_w"], "post_s": h["post_s"]}


@dataclasses.dataclass(frozen=True)
class AttnShape:
    """One attention layer of the decode step (page 'LLM decoding', "The exact architecture":
    25 sliding-window and 5 global layers, grouped-query attention; "Where the 7.36 GB goes":
    q, k and o projections, about 966M parameters). The head counts and widths are the
    reading that gives the page's count exactly: 16 query heads of 256 with 8 KV heads on
    sliding layers, 16 query heads of 512 with 2 KV heads on global ones, the cached key
    also the value. The 1024-position window is a reading too (the page gives none)."""
    hidden: int = 2816
    q_heads: int = 16
    kv_heads: int = 8
    head_dim: int = 256
    window: int = 1024       # 0: global
    capacity: int = 1032     # cache positions (a ring of window + 8 on sliding layers)
    kv_fp8: bool = False

    def params(self) -> int:
        return self.hidden * (2 * self.q_heads * self.head_dim + self.kv_heads * self.head_dim)

    def with_(self, **kw) -> "AttnShape":
        return dataclasses.replace(self, **kw)


GEMMA4_SLIDING = AttnShape()
GEMMA4_GLOBAL = AttnShape(q_heads=16, kv_heads=2, head_dim=512, window=0, capacity=32768)
GEMMA4_ATTN_LAYERS = [GEMMA4_GLOBAL if (l % 6) == 5 else GEMMA4_SLIDING for l in range(30)]   # 25 + 5, 5:1
TINY_ATTN = AttnShape(hidden=256, q_heads=4, kv_heads=2, head_dim=128, window=16, capacity=24)
KEY_STD = 1.0   # cached keys N(0, 1): the spread the projections give keys of normalised inputs


def attn_weights(shape: AttnShape, device="cpu", seed: int = 0, tag: str = "attn", layer: int = 0) -> dict:
    """FP8 q/k/o projections with per-row scales: q_w [nq dh][H], k_w [nkv dh][H],
    o_w [H][nq dh], from N(0, 0.02) like the experts."""
    H, NQ, NK = shape.hidden, shape.q_heads * shape.head_dim, shape.kv_heads * shape.head_dim
    out = {}
    out["q_w"], out["q_s"] = _fp8_matrix((NQ, H), EXPERT_STD, device, seed, tag, layer, "q")
    out["k_w"], out["k_s"] = _fp8_matrix((NK, H), EXPERT_STD, device, seed, tag, layer, "k")
    out["o_w"], out["o_s"] = _fp8_matrix((H, NQ), EXPERT_STD, device, seed, tag, layer, "o")
    return out


def kv_keys(shape: AttnShape, first_pos: int, n: int, device="cpu", seed: int = 0, tag: str = "kv",
            layer: int = 0) -> torch.Tensor:
    """Keys of positions first_pos .. first_pos + n - 1 as written into the cache: bf16
    [n][kv_heads][head_dim], N(0, KEY_STD), drawn per position so a position's key does not
    depend on n."""
    out = torch.empty((n, shape.kv_heads, shape.head_dim), dtype=torch.bfloat16, device=device)
    per = max(1, (1 << 24) // (shape.kv_heads * shape.head_dim))
    for i0 in range(0, n, per):
        i1 = min(n, i0 + per)
        for b in range((first_pos + i0) // per, (first_pos + i1 - 1) // per + 1):
            lo, hi = max(b * per, first_pos + i0), min((b + 1) * per, first_pos + i1)
            blk = normal((per, shape.kv_heads, shape.head_dim), KEY_STD, device, seed, tag, layer, b)
            out[lo - first_pos:hi - first_pos] = blk[lo - b * per:hi - b * per].to(torch.bfloat16)
    return out


def hidden_inputs(shape: Shape, M: int, step: int, sub: int = 0, device="cpu",
                  seed: int = 0, tag: str = "x") -> torch.Tensor:
    """M fresh bf16 hidden vectors N(0, 1) for one decode step (sub: resample index)."""
    return normal((M, shape.hidden), 1.0, device, seed, tag, step, sub).to(torch.bfloat16)


def stack_noise(shape: Shape, M: int, step: int, sub: int = 0, device="cpu",
                seed: int = 0) -> torch.Tensor:
    """Per-layer residual noise N(0, 0.1), bf16 [L][M][H] (stands in for attention)."""
    return normal((shape.layers, M, shape.hidden), NOISE_STD, device, seed, "noise",
                  step, sub).to(torch.bfloat16)


def rmsnorm_gains(shape: Shape, device="cpu", seed: int = 0) -> torch.Tensor:
    """bf16 gains N(1, 0.1): one per layer plus the final norm, [L + 1][H]."""
    return normal((shape.layers + 1, shape.hidden), GAIN_STD, device, seed, "gain",
                  mean=GAIN_MEAN).to(torch.bfloat16)


def zipf_router_bias(experts: int, s: float = 1.1, seed: int = 0) -> torch.Tensor:
    """Router bias that makes expert popularity Zipf-like: b_e = -s * ln(rank_e).

    rank is a seeded permutation of 1..E, so exp(b_e) is proportional to rank_e^-s.
    """
    g = _gen("cpu", seed, "zipf_rank", experts)
    rank = torch.randperm(experts, generator=g).to(torch.float64) + 1.0
    return (-s * torch.log(rank)).to(torch.float32)


def match_probability(step: int, seed: int = 0, lo: float = 0.5, hi: float = 0.9) -> float:
    """Per-step draft-match probability, uniform on [lo, hi]."""
    g = _gen("cpu", seed, "match_p", step)
    return lo + (hi - lo) * float(torch.rand((), generator=g, dtype=torch.float64))


def drafts(reference_tokens, p: float, vocab: int, step: int, seed: int = 0) -> np.ndarray:
    """gamma = len(reference_tokens) - 1 draft ids.

    Draft i (1-based) equals reference_tokens[i-1] with probability p, and is
    otherwise a uniform id different from it. reference_tokens are the tokens an
    independent run (the oracle) produced for this step, so the drafts never depend
    on the code under test.
    """
    ref = np.asarray(reference_tokens, dtype=np.int64)
    gamma = len(ref) - 1
    g = _gen("cpu", seed, "drafts", step)
    coin = torch.rand((max(gamma, 1),), generator=g, dtype=torch.float64).numpy()
    other = torch.randint(0, vocab - 1, (max(gamma, 1),), generator=g).numpy()
    out = np.empty(gamma, dtype=np.int32)
    for i in range(gamma):
        if coin[i] < p:
            out[i] = ref[i]
        else:  # uniform over the vocab minus ref[i]
            out[i] = other[i] + (1 if other[i] >= ref[i] else 0)
    return out


def bits16(t: torch.Tensor) -> np.ndarray:
    """Host numpy uint16 view of a bf16 tensor's bits."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def bytes8(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").contiguous().view(torch.uint8).numpy()


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").contiguous().to(torch.float32).numpy()


def weights_to_host(w: dict) -> dict:
    """Numpy copies of a layer_weights() dict (bf16 as uint16 bits, FP8 as uint8)."""
    out = {}
    for k, v in w.items():
        if isinstance(v, torch.Tensor):
            if v.dtype == torch.bfloat16:
                out[k] = bits16(v)
            elif v.dtype == torch.uint8:
                out[k] = bytes8(v)
            else:
                out[k] = f32(v)
        else:
            out[k] = v
    return out
