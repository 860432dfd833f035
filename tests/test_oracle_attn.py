"""Pins of the oracle's attention decode with a KV cache (oracle_attn_decode, the FP8 KV
quantiser), against what the page and the mathematics fix:
- the page's attention budget: 25 sliding and 5 global layers of q/k/o projections hold
  about 966M parameters, 1.93 GB in bf16 (page "LLM decoding", "Where the 7.36 GB goes");
- the E4M3FN quantiser against torch's float8_e4m3fn conversion, exhaustively on every
  code, every midpoint between neighbouring codes, and saturation;
- the layer against a dense numpy evaluation (projections, masked softmax, the key as value,
  the output projection), for bf16 and FP8 caches, sliding and global, M = 1..5;
- closed forms: one visible position gives o = that key; identical keys give o = the key;
  a window of 1 shows each token only its own key;
- masks: keys outside a token's window or after it do not change its output, keys inside do;
  the verify batch equals M single-token calls with the earlier keys in the history.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

FP8_TABLE = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def bf16_np(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_rne_np(v):
    v = np.asarray(v, np.float64)
    _, e = np.frexp(v)
    ex = np.maximum(e - 1, -126)
    q = np.ldexp(1.0, ex - 7)
    r = np.where(v == 0, v, np.round(v / q) * q)
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_page_attention_parameter_budget():
    """page 'LLM decoding', "Where the 7.36 GB goes": q/k/o projections under grouped-query
    attention, 25 sliding layers plus 5 global, about 966M parameters, 1.93 GB in bf16."""
    layers = synth.GEMMA4_ATTN_LAYERS
    assert sum(1 for s in layers if s.window == 0) == 5 and len(layers) == 30
    n = sum(s.params() for s in layers)
    assert n == 966_000_640
    assert round(2 * n / 1e9, 2) == 1.93


def test_fp8_quantiser_round_trips_every_code():
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            assert oracle.fp8_from_f32(float("nan")) == 0x7F
            continue
        assert oracle.fp8_from_f32(FP8_TABLE[c]) == c, c


def test_fp8_quantiser_matches_torch_on_midpoints_and_neighbours():
    vals = np.array(sorted(set(FP8_TABLE[(np.arange(256) & 0x7F) != 0x7F])))
    mids = (vals[:-1] + vals[1:]) / 2
    eps = np.float32(1e-3)
    probe = np.concatenate([mids, mids * (1 + eps), mids * (1 - eps), vals]).astype(np.float32)
    probe = probe[np.abs(probe) <= 448]
    ref = torch.from_numpy(probe).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.fp8_from_f32(v) for v in probe], np.uint8)
    # torch keeps the sign of a zero result; so does the oracle
    assert (got == ref).all(), probe[got != ref][:8]


def test_fp8_quantiser_saturates():
    for v in (448.0, 449.0, 463.9, 464.0, 480.0, 1e6, float("inf")):
        assert oracle.fp8_from_f32(v) == 0x7E and oracle.fp8_from_f32(-v) == 0xFE


def test_fp8_kv_row_scale_and_zero_row():
    rng = np.random.default_rng(1)
    x = bf16_rne_np(rng.standard_normal((6, 64)))
    codes, sc = oracle.fp8_quant_rows(x)
    xf = bf16_np(x)
    amax = np.abs(xf).max(axis=1)
    assert (sc == (amax.astype(np.float32) / np.float32(448))).all()
    # the largest element lands on +-448
    for i in range(6):
        j = np.argmax(np.abs(xf[i]))
        assert codes[i, j] & 0x7F == 0x7E
    dec = FP8_TABLE[codes] * sc[:, None]
    assert np.abs(dec - xf).max() <= (amax / 448 * 16).max()     # within half a step at the top binade
    z, zs = oracle.fp8_quant_rows(np.zeros((1, 32), np.uint16))
    assert (z == 0).all() and zs[0] == 0


def _numpy_layer(u, w, shape, M, pos, hist_keys):
    """Dense numpy evaluation of the attention layer, written from the definition."""
    H, nq, nkv, dh = shape.hidden, shape.q_heads, shape.kv_heads, shape.head_dim
    G = nq // nkv
    uf = bf16_np(u)
    Wq = FP8_TABLE[w["q_w"]] * w["q_s"].astype(np.float64)[:, None]
    Wk = FP8_TABLE[w["k_w"]] * w["k_s"].astype(np.float64)[:, None]
    Wo = FP8_TABLE[w["o_w"]] * w["o_s"].astype(np.float64)[:, None]
    q = bf16_np(bf16_rne_np(uf @ Wq.T)).reshape(M, nq, dh)
    kb = bf16_rne_np(uf @ Wk.T).reshape(M, nkv, dh)
    allk = np.concatenate([np.asarray(hist_keys, np.uint16).reshape(-1, nkv, dh), kb], axis=0)
    if shape.kv_fp8:
        codes = np.zeros(allk.shape, np.uint8)
        scales = np.zeros(allk.shape[:2], np.float32)
        for p in range(allk.shape[0]):
            for g in range(nkv):
                row = bf16_np(allk[p, g]).astype(np.float32)
                s = np.float32(np.abs(row).max()) / np.float32(448)
                scales[p, g] = s
                codes[p, g] = torch.from_numpy(row / s if s > 0 else row * 0).to(torch.float8_e4m3fn).view(
                    torch.uint8).numpy()
        keys = FP8_TABLE[codes] * scales.astype(np.float64)[..., None]
    else:
        keys = bf16_np(allk)
    o = np.zeros((M, nq, dh))
    for m in range(M):
        pm = pos + m
        lo = max(0, pm - shape.window + 1) if shape.window else 0
        for h in range(nq):
            K = keys[lo:pm + 1, h // G]
            s = K @ q[m, h] / math.sqrt(dh)
            e = np.exp(s - s.max())
            o[m, h] = (e / e.sum()) @ K
    ob = bf16_rne_np(o.reshape(M, nq * dh))
    out = bf16_np(ob) @ Wo.T
    return ob, out, kb


def _case(shape, M, pos, seed):
    w = {k: (synth.bytes8(v) if v.dtype == torch.uint8 else synth.f32(v))
         for k, v in synth.attn_weights(shape, seed=seed).items()}
    u = synth.bits16(torch.randn(M, shape.hidden, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16))
    hist = synth.bits16(synth.kv_keys(shape, 0, pos, seed=seed)) if pos else np.zeros((0, shape.kv_heads,
                                                                                      shape.head_dim), np.uint16)
    return w, u, hist


@pytest.mark.parametrize("kv_fp8", [False, True])
@pytest.mark.parametrize("window,M,pos", [(16, 1, 40), (16, 5, 40), (0, 1, 30), (0, 4, 30), (16, 3, 2), (0, 2, 0)])
def test_attn_against_dense_numpy(kv_fp8, window, M, pos):
    shape = synth.TINY_ATTN.with_(window=window, kv_fp8=kv_fp8, capacity=64)
    w, u, hist = _case(shape, M, pos, 3)
    r = oracle.attn_decode(u, w, shape, M, pos, hist)
    ob, out, kb = _numpy_layer(u, w, shape, M, pos, hist)
    assert (r["k"] == kb.reshape(M, -1)).all()
    # o and out: the same definition evaluated in a different order; bf16 results may differ
    # by one unit where the fp64 value sits on a rounding boundary
    assert (r["o_bf16"] == ob).mean() > 0.995
    np.testing.assert_allclose(r["o"].reshape(M, -1), bf16_np(ob), rtol=1e-2, atol=1e-2)
    np.testing.assert_allclose(r["out"], out, rtol=1e-6, atol=1e-6 * np.abs(out).max())


def test_single_visible_position_returns_that_key():
    shape = synth.TINY_ATTN.with_(window=1, capacity=64)
    w, u, hist = _case(shape, 3, 10, 5)
    r = oracle.attn_decode(u, w, shape, 3, 10, hist)
    G = shape.q_heads // shape.kv_heads
    o = r["o_bf16"].reshape(3, shape.q_heads, shape.head_dim)
    k = r["k"].reshape(3, shape.kv_heads, shape.head_dim)
    for h in range(shape.q_heads):
        assert (o[:, h] == k[:, h // G]).all()


def test_first_token_of_a_sequence_returns_its_key():
    shape = synth.TINY_ATTN.with_(window=0, capacity=64)
    w, u, hist = _case(shape, 1, 0, 6)
    r = oracle.attn_decode(u, w, shape, 1, 0, hist)
    G = shape.q_heads // shape.kv_heads
    o = r["o_bf16"].reshape(shape.q_heads, shape.head_dim)
    k = r["k"].reshape(shape.kv_heads, shape.head_dim)
    for h in range(shape.q_heads):
        assert (o[h] == k[h // G]).all()


def test_identical_keys_give_that_key():
    """Identical history keys and new keys equal to them (forced through a zero k projection
    and zero history): every head's output is that key, whatever the weights of the softmax."""
    shape = synth.TINY_ATTN.with_(window=0, capacity=64)
    w, u, _ = _case(shape, 2, 12, 7)
    w["k_s"] = np.zeros_like(w["k_s"])            # new keys are all zero
    hist = np.zeros((12, shape.kv_heads, shape.head_dim), np.uint16)
    r = oracle.attn_decode(u, w, shape, 2, 12, hist)
    assert (r["o_bf16"] == 0).all() and (r["out"] == 0).all()


@pytest.mark.parametrize("window", [16, 0])
def test_masks_keys_outside_the_window_or_after_the_token_do_not_count(window):
    shape = synth.TINY_ATTN.with_(window=window, capacity=64)
    M, pos = 3, 30
    w, u, hist = _case(shape, M, pos, 8)
    base = oracle.attn_decode(u, w, shape, M, pos, hist)
    lo0 = max(0, pos - window + 1) if window else 0
    if window:
        far = hist.copy()
        far[:lo0] ^= 0x0101          # outside every token's window
        r = oracle.attn_decode(u, w, shape, M, pos, far)
        assert (r["o"] == base["o"]).all()
    near = hist.copy()
    near[lo0] ^= 0x0101               # inside token 0's window
    r = oracle.attn_decode(u, w, shape, M, pos, near)
    assert not (r["o"][0] == base["o"][0]).all()


@pytest.mark.parametrize("kv_fp8", [False, True])
@pytest.mark.parametrize("window", [16, 0])
def test_verify_batch_equals_sequential_single_tokens(kv_fp8, window):
    """Token m of an M-token call sees exactly the history and tokens 0..m: the same output as
    a one-token call at pos + m whose history holds the earlier tokens' keys."""
    shape = synth.TINY_ATTN.with_(window=window, kv_fp8=kv_fp8, capacity=64)
    M, pos = 4, 25
    w, u, hist = _case(shape, M, pos, 9)
    batch = oracle.attn_decode(u, w, shape, M, pos, hist)
    kb = batch["k"].reshape(M, shape.kv_heads, shape.head_dim)
    for m in range(M):
        h = np.concatenate([hist, kb[:m]], axis=0)
        one = oracle.attn_decode(u[m:m + 1], w, shape, 1, pos + m, h)
        assert (one["o"][0] == batch["o"][m]).all()
        assert (one["out_bf16"][0] == batch["out_bf16"][m]).all()


def test_history_offset_reads_only_the_window():
    shape = synth.TINY_ATTN.with_(window=16, capacity=64)
    M, pos = 2, 50
    w, u, hist = _case(shape, M, pos, 10)
    full = oracle.attn_decode(u, w, shape, M, pos, hist)
    h0 = pos - shape.window + 1
    part = oracle.attn_decode(u, w, shape, M, pos, hist[h0:], h0=h0)
    assert (part["o"] == full["o"]).all()
    with pytest.raises(ValueError):
        oracle.attn_decode(u, w, shape, M, pos, hist[h0 + 1:], h0=h0 + 1)
