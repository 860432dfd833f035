"""Pins of the oracle's MTP drafter step (no GPU): its dense FP8 matrix-vector product and
dense GELU-gated MLP against dense numpy, and the whole chain of drafts against an
independent numpy evaluation of the same reading (page "LLM decoding", "The one-line
shape bug that disabled the model's own drafter": 5632 = 2 x 2816 -> 1024 pre_projection,
the head's own 1024-wide table; the body is a reading)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

FP8 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def bf(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rne(v):
    v = np.asarray(v, np.float64)
    _, e = np.frexp(v)
    q = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)
    r = np.where(v == 0, v, np.round(v / q) * q)
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def gelu(z):
    return torch.nn.functional.gelu(torch.from_numpy(z), approximate="tanh").numpy()


def test_gemv_and_mlp_vs_numpy():
    rng = np.random.default_rng(0)
    Q = rng.integers(0, 256, size=(64, 512), dtype=np.uint8)
    Q[(Q & 0x7F) == 0x7F] = 0x30                      # no NaN codes
    s = rng.random(64).astype(np.float32)
    x = rne(rng.normal(size=512))
    np.testing.assert_allclose(oracle.gemv_fp8(Q, s, x), (FP8[Q] @ bf(x)) * s, rtol=1e-12, atol=1e-12)
    w = synth.draft_head(synth.TINY_HEAD, seed=1)
    h = synth.draft_head_to_host(w, synth.TINY_HEAD)
    b = h["blocks"][0]
    u = rne(rng.normal(size=256))
    G = FP8[b["gate_w"]] * b["gate_s"][:, None]
    U = FP8[b["up_w"]] * b["up_s"][:, None]
    Dn = FP8[b["down_w"]] * b["down_s"][:, None]
    ref = Dn @ (gelu(G @ bf(u)) * (U @ bf(u)))
    np.testing.assert_allclose(oracle.dense_mlp(u, b["gate_w"], b["up_w"], b["down_w"], b["gate_s"], b["up_s"],
                                                b["down_s"]), ref, rtol=1e-10, atol=1e-14)


def rmsnorm(z_bits, g_bits, eps):
    z = bf(z_bits)
    r = 1.0 / math.sqrt(math.fsum(z * z) / z.size + eps)
    return rne(z * r * bf(g_bits))


def draft_numpy(tok, g, h, Qt, st, gamma, eps=1e-6):
    out, gaps = [], []
    for _ in range(gamma):
        e = rne(float(st[tok]) * FP8[Qt[tok]])
        x = np.concatenate([bf(e), bf(g)])
        z = rne((FP8[h["pre_w"]] @ x) * h["pre_s"])
        for b in h["blocks"]:
            u = bf(rmsnorm(z, b["gain"], eps))
            G = FP8[b["gate_w"]] * b["gate_s"][:, None]
            U = FP8[b["up_w"]] * b["up_s"][:, None]
            Dn = FP8[b["down_w"]] * b["down_s"][:, None]
            z = rne(bf(z) + Dn @ (gelu(G @ u) * (U @ u)))
        zf = rmsnorm(z, h["final_gain"], eps)
        lg = (FP8[h["table_w"]] @ bf(zf)) * h["table_s"]
        srt = np.sort(lg)
        tok = int(np.argmax(lg))
        gaps.append(srt[-1] - srt[-2])
        g = rne((FP8[h["post_w"]] @ bf(zf)) * h["post_s"])
        out.append(tok)
    return np.array(out), np.array(gaps)


@pytest.mark.parametrize("seed", [0, 1])
def test_draft_step_matches_numpy_chain(seed):
    sh = synth.TINY_HEAD
    h = synth.draft_head_to_host(synth.draft_head(sh, seed=seed), sh)
    tgt = synth.TINY.with_(vocab=sh.vocab)
    Qt, st = synth.lm_head(tgt, seed=seed)
    Qt, st = synth.bytes8(Qt), synth.f32(st)
    g0 = synth.bits16(synth.hidden_inputs(tgt, 1, 0, tag="draft_g"))[0]
    r = oracle.draft_step(17, g0, h, Qt, st, gamma=4)
    d, gaps = draft_numpy(17, g0, h, Qt, st, 4)
    assert (gaps > 1e-9).all()
    assert (r["drafts"] == d).all(), (r["drafts"], d)
    np.testing.assert_allclose(r["gaps"], gaps, rtol=1e-9, atol=1e-12)


def test_mtp_head_holds_about_430m_parameters():
    # page "LLM decoding", "Lever 2: fewer passes": a 430M Multi-Token-Prediction head
    assert abs(synth.MTP_HEAD.params() / 430e6 - 1) < 0.01
    assert 2 * synth.MTP_HEAD.hidden == 5632 and synth.MTP_HEAD.width == 1024   # the pre_projection, 5632 -> 1024
