"""GPU parity: every entry point of the C ABI against the CPU oracle on the same
seeded inputs. Integer results (expert ids, argmax tokens, accepted lengths) must
be bit-exact; bf16 outputs within rel-L2 2e-3 and max-abs 1e-2 of the oracle's
fp64 values. Inputs are resampled until no decision is within 1e-3 of a tie in the
oracle (fp32 accumulation error is far below that)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from fine_grained_moe_router_amd import native
from parity_util import (TAU, bf16_f64, check_bf16_output, to_device, unambiguous_layer_input,
                         unambiguous_lm_input)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ helpers

class Layer:
    """Device weights of one layer plus a host copy for the oracle."""

    def __init__(self, shape, layer=0, seed=0, device_gen="cpu", router_bias=None, expert_dtype="fp8",
                 router_dtype="bf16"):
        w = synth.layer_weights(shape, layer, device_gen, seed=seed, router_bias=router_bias,
                                expert_dtype=expert_dtype, router_dtype=router_dtype)
        self.shape = shape
        self.dev = to_device(w, DEV)
        self.host = synth.weights_to_host(w)
        self.desc = native.layer_desc(shape, expert_dtype, router_dtype)
        self.lw = native.layer_weights(self.dev)

    def run(self, x_bits_dev, M):
        sh = self.shape
        wsb = native.moe_decode_layer_workspace(self.desc, M)
        ws = native.workspace(wsb)
        y = torch.empty(M, sh.hidden, dtype=torch.bfloat16, device=DEV)
        idx = torch.full((M, sh.top_k), -7, dtype=torch.int32, device=DEV)
        wts = torch.zeros(M, sh.top_k, dtype=torch.float32, device=DEV)
        native.moe_decode_layer(self.desc, self.lw, M, x_bits_dev, y, idx, wts, ws, wsb)
        torch.cuda.synchronize()
        assert native.moe_decode_layer_status(self.desc, ws) == native.MOE_OK
        return synth.bits16(y), idx.cpu().numpy(), wts.cpu().numpy()


def check_layer(layer, x, r, what):
    M = x.shape[0]
    y, idx, wts = layer.run(x.to(DEV), M)
    assert (idx == r["idx"]).all(), "%s: expert ids differ\n%s\n%s" % (what, idx, r["idx"])
    np.testing.assert_allclose(wts, r["w"], rtol=2e-5, atol=1e-7, err_msg=what)
    return check_bf16_output(y, r["y"], r["y_bf16"], what)


# ---------------------------------------------------------------- FP8 decode

def test_fp8_decode_all_256_codes_on_device():
    codes = torch.arange(256, dtype=torch.uint8, device=DEV)
    a = torch.empty(256, dtype=torch.float32, device=DEV)
    b = torch.empty(256, dtype=torch.float32, device=DEV)
    native.moe_fp8_decode(256, codes, a, b)
    torch.cuda.synchronize()
    a, b = a.cpu().numpy(), b.cpu().numpy()
    for c in range(256):
        ref = oracle.fp8_e4m3(c)
        if np.isnan(ref):
            assert np.isnan(a[c]) and np.isnan(b[c]), c
        else:
            assert a[c] == ref and b[c] == ref, (c, a[c], b[c], ref)
            assert np.signbit(a[c]) == np.signbit(ref) and np.signbit(b[c]) == np.signbit(ref)


# ------------------------------------------------------------ one MoE layer

@pytest.mark.parametrize("M", [1, 2, 5, 8])
@pytest.mark.parametrize("seed", [0, 1])
def test_tiny_layer(M, seed):
    sh = synth.TINY
    say("tiny layer M=%d seed=%d" % (M, seed))
    L = Layer(sh, seed=seed)
    for step in range(3):
        x, r = unambiguous_layer_input(sh, M, L.host, step + 10 * seed)
        check_layer(L, x, r, "tiny M=%d seed=%d step=%d" % (M, seed, step))


VARIANTS = {
    "no_shared": synth.TINY.with_(shared_width=0),
    "wide_shared": synth.TINY.with_(shared_width=192),
    "top1": synth.TINY.with_(top_k=1),
    "all_experts": synth.TINY.with_(top_k=16),
    "e256_k8": synth.TINY.with_(experts=256, top_k=8, hidden=512, width=128, shared_width=64),
    "e128_k16": synth.TINY.with_(experts=128, top_k=16, hidden=768),
    "e48": synth.TINY.with_(experts=48, top_k=6),
    # E not a multiple of 8: the one-launch form gathers the router one element per load
    "e18": synth.TINY.with_(experts=18, top_k=3),
    "wide_d": synth.TINY.with_(hidden=1024, width=320, shared_width=128),
    # beyond the fused kernel's unit geometry (H > 2816, D > 704): the separate per-layer kernels
    "beyond_fused_h": synth.TINY.with_(hidden=3072, experts=16, top_k=2, width=64, shared_width=64),
    "beyond_fused_d": synth.TINY.with_(hidden=512, width=768, shared_width=128),
}


@pytest.mark.parametrize("name", sorted(VARIANTS))
@pytest.mark.parametrize("M", [1, 5, 8])
def test_layer_shape_variants(name, M):
    sh = VARIANTS[name]
    say("variant %s M=%d" % (name, M))
    L = Layer(sh, seed=3)
    x, r = unambiguous_layer_input(sh, M, L.host, 100)
    check_layer(L, x, r, "%s M=%d" % (name, M))


FP8_ROUTER_SHAPES = {"tiny": synth.TINY, "e18": VARIANTS["e18"], "e48": VARIANTS["e48"],
                     "h2816": synth.TINY.with_(hidden=2816, experts=32, top_k=4, width=704, shared_width=704)}


@pytest.mark.parametrize("name", sorted(FP8_ROUTER_SHAPES))
@pytest.mark.parametrize("M", [1, 5, 8])
def test_layer_fp8_router(name, M):
    """The precision ladder's FP8 router rung: router codes [H][E] with per-expert scales,
    gathered by the one-launch form of moe_decode_layer (16-byte tile or, for E = 18, one
    code per load)."""
    sh = FP8_ROUTER_SHAPES[name]
    say("fp8 router %s M=%d" % (name, M))
    L = Layer(sh, seed=6, router_dtype="fp8")
    x, r = unambiguous_layer_input(sh, M, L.host, 300 + M)
    check_layer(L, x, r, "fp8 router %s M=%d" % (name, M))


def test_layer_fp8_router_needs_the_one_launch_form():
    """The separate per-layer kernels read a bf16 router: a layer beyond the fused geometry
    with an FP8 router is refused (no workspace size, MOE_EUNSUPPORTED)."""
    d = native.layer_desc(VARIANTS["beyond_fused_d"], "fp8", "fp8")
    assert native.moe_decode_layer_workspace(d, 1) == 0


def test_layer_with_zipf_router_bias():
    sh = synth.TINY.with_(experts=64, top_k=4, hidden=512)
    L = Layer(sh, seed=4, router_bias=synth.zipf_router_bias(64))
    for M in (1, 8):
        x, r = unambiguous_layer_input(sh, M, L.host, 200)
        check_layer(L, x, r, "zipf M=%d" % M)


BF16_SHAPES = {
    "tiny": synth.TINY,
    "tiny_wide_shared": synth.TINY.with_(shared_width=192),
    "h2816": synth.TINY.with_(hidden=2816, experts=32, top_k=4, width=704, shared_width=704),
}


@pytest.mark.parametrize("name", sorted(BF16_SHAPES))
@pytest.mark.parametrize("M", [1, 5, 8])
def test_layer_bf16_experts(name, M):
    """bf16 expert weights (no scales): the same layer arithmetic with the weights used
    as they are."""
    sh = BF16_SHAPES[name]
    say("bf16 experts %s M=%d" % (name, M))
    L = Layer(sh, seed=6, expert_dtype="bf16")
    x, r = unambiguous_layer_input(sh, M, L.host, 300 + M)
    check_layer(L, x, r, "bf16 %s M=%d" % (name, M))


def test_layer_bf16_experts_with_zipf_router_bias():
    sh = synth.TINY.with_(experts=64, top_k=4, hidden=512)
    L = Layer(sh, seed=7, router_bias=synth.zipf_router_bias(64), expert_dtype="bf16")
    for M in (1, 8):
        x, r = unambiguous_layer_input(sh, M, L.host, 400)
        check_layer(L, x, r, "bf16 zipf M=%d" % M)


def test_batch_consistency_identical_tokens_and_determinism():
    sh = synth.TINY.with_(experts=64, top_k=4, hidden=512, width=128)
    L = Layer(sh, seed=5)
    x = synth.hidden_inputs(sh, 5, 0).to(DEV)
    y5, i5, w5 = L.run(x, 5)
    for m in range(5):
        y1, i1, w1 = L.run(x[m:m + 1].contiguous(), 1)
        assert (y1[0] == y5[m]).all() and (i1[0] == i5[m]).all() and (w1[0] == w5[m]).all(), m
    xr = x[2:3].repeat(8, 1).contiguous()
    y8, i8, _ = L.run(xr, 8)
    assert (y8 == y8[0]).all() and (i8 == i8[0]).all() and (y8[0] == y5[2]).all()
    y5b, i5b, w5b = L.run(x, 5)
    assert (y5b == y5).all() and (i5b == i5).all() and (w5b == w5).all()


@pytest.fixture(scope="module")
def gemma_layer():
    sh = synth.GEMMA4_26B_A4B.with_(layers=1)
    say("generating one Gemma-4-26B-A4B-shaped layer")
    return Layer(sh, layer=0, seed=0, device_gen=DEV)


@pytest.mark.parametrize("M,steps", [(1, 12), (5, 4), (8, 2)])
def test_gemma_layer(gemma_layer, M, steps):
    sh = gemma_layer.shape
    worst = 0.0
    for step in range(steps):
        say("gemma layer M=%d step=%d" % (M, step))
        x, r = unambiguous_layer_input(sh, M, gemma_layer.host, 1000 + step)
        err, _ = check_layer(gemma_layer, x, r, "gemma M=%d step=%d" % (M, step))
        worst = max(worst, err)
    say("worst rel-L2 %.3g" % worst)


def test_gemma_layer_batch_consistency(gemma_layer):
    sh = gemma_layer.shape
    x = synth.hidden_inputs(sh, 5, 77).to(DEV)
    y5, i5, _ = gemma_layer.run(x, 5)
    for m in range(5):
        y1, i1, _ = gemma_layer.run(x[m:m + 1].contiguous(), 1)
        assert (y1[0] == y5[m]).all() and (i1[0] == i5[m]).all(), m


def test_gemma_layer_shared_2112(gemma_layer):
    # the page's dense MLP width for the shared expert
    sh = synth.GEMMA4_26B_A4B.with_(layers=1, shared_width=2112, experts=32)
    L = Layer(sh, seed=6, device_gen=DEV)
    for M in (1, 8):
        x, r = unambiguous_layer_input(sh, M, L.host, 300 + M)
        check_layer(L, x, r, "shared2112 M=%d" % M)


@pytest.mark.parametrize("where", ["gemma", "tiny_fp8_router", "e18_fp8_router"])
@pytest.mark.parametrize("M", [1, 5, 8])
def test_layer_expert_major_router_is_bit_identical(gemma_layer, where, M):
    """MOE_ROUTER_EXPERT_MAJOR: the same router values passed [E][H] (transposed on the
    device) give the same expert ids, weights and y bit for bit as the [H][E] call, since the
    router workgroups then hold the same values in the same lanes; E = 18 covers rows that
    are not 16-byte aligned in the [H][E] layout."""
    if where == "gemma":
        L, rdt = gemma_layer, "bf16"
    else:
        rdt = "fp8"
        L = Layer(synth.TINY if where.startswith("tiny") else VARIANTS["e18"], seed=6, router_dtype="fp8")
    sh = L.shape
    em = dict(L.dev)
    em["router_w"] = L.dev["router_w"].t().contiguous()
    desc = native.layer_desc(sh, "fp8", rdt, expert_major=True)
    lw = native.layer_weights(em)
    x = synth.hidden_inputs(sh, M, 600 + M).to(DEV)
    y0, i0, w0 = L.run(x, M)
    wsb = native.moe_decode_layer_workspace(desc, M)
    ws = native.workspace(wsb)
    y = torch.empty(M, sh.hidden, dtype=torch.bfloat16, device=DEV)
    idx = torch.full((M, sh.top_k), -7, dtype=torch.int32, device=DEV)
    wts = torch.zeros(M, sh.top_k, dtype=torch.float32, device=DEV)
    native.moe_decode_layer(desc, lw, M, x, y, idx, wts, ws, wsb)
    torch.cuda.synchronize()
    assert native.moe_decode_layer_status(desc, ws) == native.MOE_OK
    say("%s M=%d: expert-major router" % (where, M))
    assert (idx.cpu().numpy() == i0).all() and (wts.cpu().numpy() == w0).all()
    assert (synth.bits16(y) == y0).all()


def _unit_rms_inputs(shape, M, seed):
    """bf16 +-1 vectors: with unit gains and eps 0 their RMSNorm is themselves."""
    g = torch.Generator().manual_seed(seed)
    sign = torch.randint(0, 2, (M, shape.hidden), generator=g) * 2 - 1
    return sign.to(torch.bfloat16)


@pytest.mark.parametrize("where", ["tiny", "gemma", "tiny_fp8_router"])
@pytest.mark.parametrize("M", [1, 5, 8])
def test_layer_entry_point_is_bit_identical_to_the_fused_step_layer(gemma_layer, where, M):
    """moe_decode_layer and the fused step's layer share the routing, the units and the
    combine: on the same normalised input they give the same expert ids and weights and
    the same y bit for bit. The fused step normalises its input itself; with +-1 inputs,
    unit gains and eps 0 that norm returns the input unchanged, so both see the same u."""
    from fine_grained_moe_router_amd.stack import FusedDecodeStep
    if where == "gemma":
        layer = gemma_layer
    elif where == "tiny_fp8_router":   # the router gathered from [H][E] vs the prepared [E][H] copy
        layer = Layer(synth.TINY, seed=12, router_dtype="fp8")
    else:
        layer = Layer(synth.TINY, seed=12)
    sh = layer.shape.with_(layers=1)
    x = _unit_rms_inputs(sh, M, 77 + M)
    xd = x.to(DEV)
    y_l, i_l, w_l = layer.run(xd, M)
    gains = torch.ones(2, sh.hidden, dtype=torch.bfloat16, device=DEV)
    Q, s = synth.lm_head(sh.with_(vocab=4096), DEV, seed=1)
    fs = FusedDecodeStep(sh.with_(vocab=4096), [layer.dev], gains, Q, s, max_M=8, eps=0.0)
    noise = torch.zeros(1, M, sh.hidden, dtype=torch.bfloat16, device=DEV)
    d = torch.zeros(max(M - 1, 1), dtype=torch.int32, device=DEV)
    fs.step(xd, noise, d if M > 1 else None, M)
    torch.cuda.synchronize()
    assert fs.status() == native.MOE_OK
    assert (fs.topk_idx(M)[0].cpu().numpy() == i_l).all()
    assert (fs.topk_w(M)[0].cpu().numpy().view(np.uint32) == w_l.view(np.uint32)).all()
    assert (synth.bits16(fs.y(M)[0]) == y_l).all(), "%s M=%d: y differs between the two entry points" % (where, M)
    # and both against the oracle, where its routing margins allow a one-to-one comparison
    r = oracle.moe_layer(synth.bits16(x), layer.host, sh.top_k)
    if (r["gap"] >= TAU).all():
        assert (i_l == r["idx"]).all()
        check_bf16_output(y_l, r["y"], None, "%s M=%d" % (where, M))


# ----------------------------------------------------------------- lm_head

def run_lm(Q, s, x, V, H):
    M = x.shape[0]
    wsb = native.lm_head_argmax_workspace(M, H, V)
    ws = native.workspace(wsb)
    tok = torch.full((M,), -3, dtype=torch.int32, device=DEV)
    ml = torch.zeros(M, dtype=torch.float32, device=DEV)
    native.lm_head_argmax(M, H, V, x, Q, s, tok, ml, ws, wsb)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), ml.cpu().numpy()


@pytest.mark.parametrize("M", [1, 5, 8])
def test_lm_head_tiny(M):
    sh = synth.TINY
    Q, s = synth.lm_head(sh)
    Qh, sh_ = synth.bytes8(Q), synth.f32(s)
    Qd, sd = Q.to(DEV), s.to(DEV)
    for step in range(3):
        x, tok, ml = unambiguous_lm_input(sh, M, Qh, sh_, step)
        t, m = run_lm(Qd, sd, x.to(DEV), sh.vocab, sh.hidden)
        assert (t == tok).all(), (t, tok)
        np.testing.assert_allclose(m, ml, rtol=1e-5, atol=1e-6)


def test_lm_head_ties_go_to_lower_id():
    sh = synth.TINY
    Q, s = synth.lm_head(sh)
    x = synth.hidden_inputs(sh, 2, 5)
    xs = bf16_f64(synth.bits16(x[0]))
    Q = Q.clone()
    s = s.clone()
    row = torch.from_numpy(np.where(xs >= 0, 0x7E, 0xFE).astype(np.uint8))
    for v in (3000, 1234, 4000):       # three identical winning rows
        Q[v] = row
        s[v] = 1.0
    t, _ = run_lm(Q.to(DEV), s.to(DEV), x.to(DEV), sh.vocab, sh.hidden)
    assert t[0] == 1234


@pytest.fixture(scope="module")
def gemma_lm_head():
    sh = synth.GEMMA4_26B_A4B
    say("generating the 262144 x 2816 lm_head")
    Q, s = synth.lm_head(sh, DEV)
    return sh, Q, s, synth.bytes8(Q), synth.f32(s)


@pytest.mark.parametrize("M", [1, 5])
def test_lm_head_full_size(gemma_lm_head, M):
    sh, Q, s, Qh, shh = gemma_lm_head
    say("full lm_head M=%d" % M)
    x, tok, ml = unambiguous_lm_input(sh, M, Qh, shh, 7 + M)
    t, m = run_lm(Q, s, x.to(DEV), sh.vocab, sh.hidden)
    assert (t == tok).all(), (t, tok)
    np.testing.assert_allclose(m, ml, rtol=1e-5, atol=1e-6)


# -------------------------------------------------------------- acceptance

@pytest.mark.parametrize("full", [False, True])
@pytest.mark.parametrize("M", [1, 5])
def test_lm_head_bf16(M, full):
    """The precision ladder's BF16 lm_head rung: bf16 weights, no scales."""
    sh = synth.GEMMA4_26B_A4B if full else synth.TINY
    W = synth.lm_head_bf16(sh, DEV if full else "cpu", seed=4)
    Wh = synth.bits16(W)
    for sub in range(50):
        x = synth.hidden_inputs(sh, M, 60, sub, tag="lmbf")
        tok, ml, gap = oracle.lm_head_argmax_bf16(synth.bits16(x), Wh)
        if (gap >= TAU).all():
            break
    wsb = native.lm_head_argmax_workspace(M, sh.hidden, sh.vocab)
    ws = native.workspace(wsb)
    t = torch.empty(M, dtype=torch.int32, device=DEV)
    mlg = torch.empty(M, dtype=torch.float32, device=DEV)
    native.lm_head_argmax_bf16(M, sh.hidden, sh.vocab, x.to(DEV), W.to(DEV), t, mlg, ws, wsb)
    torch.cuda.synchronize()
    assert (t.cpu().numpy() == tok).all()
    np.testing.assert_allclose(mlg.cpu().numpy(), ml, rtol=1e-5, atol=1e-6)


def test_spec_accept_all_patterns():
    rng = np.random.default_rng(0)
    for gamma in range(8):
        for pat in range(1 << gamma):
            target = rng.integers(0, 262144, gamma + 1).astype(np.int32)
            draft = np.array([target[i] if (pat >> i) & 1 else (target[i] + 1 + i) % 262144
                              for i in range(gamma)], np.int32)
            n_ref, out_ref = oracle.spec_accept(draft, target)
            d = torch.from_numpy(draft if gamma else np.zeros(1, np.int32)).to(DEV)
            t = torch.from_numpy(target).to(DEV)
            n = torch.full((4,), -9, dtype=torch.int32, device=DEV)
            out = torch.full((gamma + 1,), -9, dtype=torch.int32, device=DEV)
            native.spec_accept(gamma, d if gamma else None, t, n, out)
            torch.cuda.synchronize()
            assert int(n[0]) == n_ref and (out.cpu().numpy() == out_ref).all(), (gamma, pat)


# ------------------------------------------------------------ add + RMSNorm

@pytest.mark.parametrize("H", [256, 2816])
@pytest.mark.parametrize("M", [1, 5, 8])
def test_add_rmsnorm(H, M):
    sh = synth.TINY.with_(hidden=H, layers=1)
    h = synth.hidden_inputs(sh, M, 1, tag="h")
    a0 = synth.stack_noise(sh, M, 1)[0]
    a1 = synth.hidden_inputs(sh, M, 2, tag="a1")
    g = synth.rmsnorm_gains(sh)[0]
    ho_ref, u_ref = oracle.add_rmsnorm(synth.bits16(h), synth.bits16(a0), synth.bits16(a1), synth.bits16(g))
    for with_a1 in (True, False):
        if not with_a1:
            ho_ref, u_ref = oracle.add_rmsnorm(synth.bits16(h), synth.bits16(a0), None, synth.bits16(g))
        hd = h.to(DEV)
        ho = torch.empty_like(hd)
        u = torch.empty_like(hd)
        native.moe_add_rmsnorm(M, H, hd, a0.to(DEV), a1.to(DEV) if with_a1 else None, g.to(DEV), 1e-6, ho, u)
        torch.cuda.synchronize()
        hb, ub = synth.bits16(ho), synth.bits16(u)
        assert (np.abs(hb.astype(np.int32) - ho_ref.astype(np.int32)) <= 1).all()
        assert (hb == ho_ref).mean() > 0.999
        # u is itself a bf16 rounding: compare bit patterns (at most one ulp apart, almost all equal)
        assert (np.abs(ub.astype(np.int32) - u_ref.astype(np.int32)) <= 1).all()
        assert (ub == u_ref).mean() > 0.99
        # in place (h_out == h_in) gives the same bits
        hd2 = h.to(DEV)
        u2 = torch.empty_like(hd2)
        native.moe_add_rmsnorm(M, H, hd2, a0.to(DEV), a1.to(DEV) if with_a1 else None, g.to(DEV), 1e-6, hd2, u2)
        torch.cuda.synchronize()
        assert (synth.bits16(hd2) == hb).all() and (synth.bits16(u2) == ub).all()


def test_hbm_read_probe_reads_every_byte_once():
    """The read probe's sink words XOR to the XOR of every 32-bit word of the buffer (each
    16-byte piece is read exactly once), including a tail that is not a multiple of the
    grid's stride."""
    g = torch.Generator().manual_seed(11)
    for nbytes in (16, 4096 * 256 * 16 * 4 + 48, 3 << 20):
        data = torch.randint(0, 2 ** 31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32)
        src = data.to(DEV)
        sink = torch.zeros(native.PROBE_GRID, dtype=torch.int32, device=DEV)
        native.moe_hbm_read_probe(src, nbytes, sink)
        torch.cuda.synchronize()
        want = np.bitwise_xor.reduce(data.numpy().view(np.uint32))
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == want, nbytes

