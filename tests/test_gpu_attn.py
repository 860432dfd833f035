"""GPU parity of the attention decode with a KV cache (moe_kv_cache_write, moe_attn_decode)
against the oracle's attention layer, through the C ABI.

- The FP8 cache rows the write call stores for the history keys: codes and scales bit for
  bit against the oracle's quantiser on the same bf16 keys (the decision is the same fp32
  division and round-to-nearest-even on both sides).
- The layer: the new keys as the bf16 cache stores them (one bf16 ulp at most, almost all
  identical), the heads' outputs o and the output out against the oracle's bf16 values
  within rel-L2 2e-3 and, per element, 1e-2 or one bf16 step of the value where that is
  larger (the bar of the MoE layer's y: bf16 vectors, fp32 accumulation against fp64; the
  two sides' bf16 roundings agree but where the fp64 value sits near a rounding boundary,
  and above 2 one step is 2^-6).
- Shapes: a tiny layer (sliding with the ring wrapped, and global), and the Gemma-4-26B-A4B
  sliding (16 x 256, 8 KV heads, window 1024) and global (16 x 512, 2 KV heads) layers at
  long contexts, M = 1, 5 and 8 (the global layer also at M = 2 and 3 and at its first
  positions), bf16 and FP8 caches. 512-wide heads with up to 64 queries per KV head, and
  256-wide heads with 8 to 64, run the partial softmax on the matrix cores (one to four query
  tiles); a layer with 16 query heads per KV head at M = 5 (80 queries) and the sliding layer
  below 8 queries per KV head run it on the vector units, and a 512-wide sliding layer checks
  the matrix-core path's window and ring. Determinism of both paths.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from fine_grained_moe_router_amd import native

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def relerr(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30)


def bf(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def close_bf16(got_bits, ref_bits):
    """Every element within 1e-2 of the reference, or within one bf16 step of it where that
    step is larger (values of magnitude 2 and more: a sum that lies near a rounding boundary
    can round to either neighbour, and the neighbours are 2^-6 apart there)."""
    g, r = bf(got_bits), bf(ref_bits)
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(r), 1e-30))) - 7)
    return bool((np.abs(g - r) <= np.maximum(1e-2, step)).all())


def run_layer(shape, M, pos, seed, h0=None):
    """Fill the cache with the history keys of positions h0 .. pos - 1, run one decode call,
    return the GPU results, the cache and the oracle's results."""
    if h0 is None:
        h0 = max(0, pos - shape.window + 1) if shape.window else 0
    desc = native.attn_desc(shape)
    w = synth.attn_weights(shape, DEV, seed=seed)
    wd = native.attn_weights(w)
    cache = native.workspace(native.moe_kv_cache_bytes(desc))
    hist = synth.kv_keys(shape, h0, pos - h0, DEV, seed=seed) if pos > h0 else None
    if hist is not None:
        native.moe_kv_cache_write(desc, h0, pos - h0, hist.contiguous(), cache)
    u = synth.hidden_inputs(synth.GEMMA4_26B_A4B.with_(hidden=shape.hidden), M, 0, device=DEV, seed=seed,
                            tag="attn_u").contiguous()
    out = torch.empty(M, shape.hidden, dtype=torch.bfloat16, device=DEV)
    o = torch.empty(M, shape.q_heads * shape.head_dim, dtype=torch.bfloat16, device=DEV)
    wsb = native.moe_attn_decode_workspace(desc, M)
    ws = native.workspace(wsb)
    native.moe_attn_decode(desc, wd, M, pos, u, cache, out, o, ws, wsb)
    torch.cuda.synchronize()
    host = {k: (synth.bytes8(v) if v.dtype == torch.uint8 else synth.f32(v)) for k, v in w.items()}
    hk = synth.bits16(hist) if hist is not None else np.zeros((0, shape.kv_heads, shape.head_dim), np.uint16)
    r = oracle.attn_decode(synth.bits16(u), host, shape, M, pos, hk, h0=h0)
    return {"out": synth.bits16(out), "o": synth.bits16(o), "cache": cache, "hist": hk, "h0": h0}, r


def cache_views(shape, cache):
    """(values, scales) of a cache buffer: bf16 bits or FP8 codes [kv_heads][capacity][head_dim]."""
    n = shape.kv_heads * shape.capacity * shape.head_dim
    c = cache.cpu().numpy()
    if not shape.kv_fp8:
        return c[:2 * n].view(np.uint16).reshape(shape.kv_heads, shape.capacity, shape.head_dim), None
    off = (n + 255) // 256 * 256
    codes = c[:n].reshape(shape.kv_heads, shape.capacity, shape.head_dim)
    scales = c[off:off + 4 * shape.kv_heads * shape.capacity].view(np.float32).reshape(shape.kv_heads, shape.capacity)
    return codes, scales


def check(shape, M, pos, g, r, tag):
    e_o, e_out = relerr(bf(g["o"]), bf(r["o_bf16"])), relerr(bf(g["out"]), bf(r["out_bf16"]))
    same_o, same_out = (g["o"] == r["o_bf16"]).mean(), (g["out"] == r["out_bf16"]).mean()
    say("%s M=%d pos=%d: o rel-L2 %.2e (%.4f identical), out rel-L2 %.2e (%.4f identical; %.2e against fp64)" % (
        tag, M, pos, e_o, same_o, e_out, same_out, relerr(bf(g["out"]), r["out"])))
    assert e_o <= 2e-3 and close_bf16(g["o"], r["o_bf16"])
    assert e_out <= 2e-3 and close_bf16(g["out"], r["out_bf16"])
    vals, scales = cache_views(shape, g["cache"])
    slots = [(pos + m) % shape.capacity for m in range(M)]
    newk = r["k"].reshape(M, shape.kv_heads, shape.head_dim)
    if not shape.kv_fp8:
        got = np.stack([vals[:, s] for s in slots])          # [M][kv][dh]
        assert (got == newk).mean() > 0.99
        assert np.abs(got.astype(np.int32) - newk.astype(np.int32)).max() <= 1
    else:
        dec = oracle._fp8_values()[np.stack([vals[:, s] for s in slots])] * \
            np.stack([scales[:, s] for s in slots])[..., None]
        ref = oracle._fp8_values()[r["k_codes"]] * r["k_scales"][..., None]
        assert relerr(dec, ref) <= 2e-2           # FP8 steps of keys whose bf16 values may differ by an ulp
        # the history rows: bit for bit
        if len(g["hist"]):
            codes, sc = oracle.fp8_quant_rows(g["hist"])
            for i in range(0, len(g["hist"]), max(1, len(g["hist"]) // 64)):
                s = (g["h0"] + i) % shape.capacity
                assert (vals[:, s] == codes[i]).all() and (scales[:, s] == sc[i]).all(), i


TINY_SLIDING = synth.TINY_ATTN
TINY_GLOBAL = synth.TINY_ATTN.with_(window=0, capacity=256)


@pytest.mark.parametrize("kv_fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("M,pos", [(1, 0), (1, 5), (3, 5), (5, 40), (8, 61), (1, 100)])
def test_attn_tiny_sliding_ring(kv_fp8, M, pos):
    shape = TINY_SLIDING.with_(kv_fp8=kv_fp8)
    g, r = run_layer(shape, M, pos, 11)
    check(shape, M, pos, g, r, "tiny sliding")


@pytest.mark.parametrize("kv_fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("M,pos", [(1, 0), (2, 1), (5, 17), (8, 200)])
def test_attn_tiny_global(kv_fp8, M, pos):
    shape = TINY_GLOBAL.with_(kv_fp8=kv_fp8)
    g, r = run_layer(shape, M, pos, 12)
    check(shape, M, pos, g, r, "tiny global")


@pytest.mark.parametrize("kv_fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("M", [1, 3, 4, 5, 8])
def test_attn_gemma_sliding_layer(kv_fp8, M):
    """The Gemma sliding layer with the ring wrapped several times (pos 5000, capacity 1032):
    2 and 6 queries per KV head on the vector units (M = 1, 3), 8, 10 and 16 on the matrix
    cores (M = 4, 5, 8)."""
    shape = synth.GEMMA4_SLIDING.with_(kv_fp8=kv_fp8)
    g, r = run_layer(shape, M, 5000, 13)
    check(shape, M, 5000, g, r, "gemma sliding")


@pytest.mark.parametrize("kv_fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
def test_attn_gemma_global_layer(kv_fp8, M):
    """The Gemma global layer at an 8K context (16 query heads of 512, 2 KV heads), its
    partial softmax on the matrix cores: half a query tile (M = 1), one full tile (M = 2), a
    partial second one (M = 3), three (M = 5) and four (M = 8)."""
    shape = synth.GEMMA4_GLOBAL.with_(kv_fp8=kv_fp8, capacity=8200)
    g, r = run_layer(shape, M, 8000, 14)
    check(shape, M, 8000, g, r, "gemma global")


@pytest.mark.parametrize("kv_fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("M,pos", [(1, 0), (2, 0), (5, 5), (8, 31), (5, 40), (1, 33)])
def test_attn_gemma_global_short(kv_fp8, M, pos):
    """The matrix-core path at the first positions: one or two 32-position chunks, most of
    them masked (a query sees only the positions up to its own), the new keys inside them."""
    shape = synth.GEMMA4_GLOBAL.with_(kv_fp8=kv_fp8, capacity=128)
    g, r = run_layer(shape, M, pos, 17)
    check(shape, M, pos, g, r, "gemma global short")


@pytest.mark.parametrize("kv_fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("M", [4, 5])
def test_attn_global_wide_group(kv_fp8, M):
    """512-wide heads with 16 query heads per KV head: 64 queries per KV head at M = 4 (four
    tiles on the matrix cores) and 80 at M = 5 (more than one workgroup of the matrix-core
    form holds, so the vector-unit kernel runs)."""
    shape = synth.GEMMA4_GLOBAL.with_(q_heads=32, kv_fp8=kv_fp8, capacity=2100)
    g, r = run_layer(shape, M, 2000, 18)
    check(shape, M, 2000, g, r, "global G=16")


@pytest.mark.parametrize("kv_fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("M", [1, 5])
def test_attn_512_wide_sliding(kv_fp8, M):
    """512-wide heads with a window on the matrix cores: a 300-position window over a ring of
    308 slots, wrapped several times; the masks of the window's first position and of the
    verify batch's later tokens fall inside the chunks."""
    shape = synth.GEMMA4_GLOBAL.with_(window=300, capacity=308, kv_fp8=kv_fp8)
    g, r = run_layer(shape, M, 1000, 19)
    check(shape, M, 1000, g, r, "512-wide sliding")


@pytest.mark.parametrize("kv_fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("M", [1, 8])
def test_attn_widest_call(kv_fp8, M):
    """The largest widths the call accepts: hidden 4096 and q_heads x head_dim = 16,384 (32
    heads of 512 over 2 KV heads, 16 per group). The o projection then takes 64 lanes per row
    and one token per LDS group; at M = 8 the 128 queries per KV head exceed the matrix-core
    form, so the 512-wide vector kernel runs with eight query tiles."""
    shape = synth.AttnShape(hidden=4096, q_heads=32, kv_heads=2, head_dim=512, window=0, capacity=520, kv_fp8=kv_fp8)
    g, r = run_layer(shape, M, 500, 21)
    check(shape, M, 500, g, r, "widest")


@pytest.mark.parametrize("kv_fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("M", [1, 5])
def test_attn_many_narrow_heads(kv_fp8, M):
    """The most query heads (64 of 128 over 4 KV heads, 16 per group) with a 64-position window
    on a 72-slot ring that has wrapped four times: five query tiles per KV head at M = 5."""
    shape = synth.AttnShape(q_heads=64, kv_heads=4, head_dim=128, window=64, capacity=72, kv_fp8=kv_fp8)
    g, r = run_layer(shape, M, 300, 22)
    check(shape, M, 300, g, r, "narrow heads")


def test_attn_gemma_global_full_context_fp8():
    """The last positions of a 32K-slot global cache (FP8), one token; the oracle sees every
    position, so this is the largest case it evaluates."""
    shape = synth.GEMMA4_GLOBAL.with_(kv_fp8=True)
    g, r = run_layer(shape, 1, shape.capacity - 1, 15)
    check(shape, 1, shape.capacity - 1, g, r, "gemma global 32K")


@pytest.mark.parametrize("shape", [synth.GEMMA4_SLIDING.with_(kv_fp8=True),
                                   synth.GEMMA4_GLOBAL.with_(kv_fp8=True, capacity=4096)], ids=["sliding", "global"])
def test_attn_is_deterministic(shape):
    a, _ = run_layer(shape, 5, 3000, 16)
    b, _ = run_layer(shape, 5, 3000, 16)
    assert (a["out"] == b["out"]).all() and (a["o"] == b["o"]).all()
    assert torch.equal(a["cache"], b["cache"])
