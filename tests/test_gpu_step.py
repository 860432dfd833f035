"""GPU parity of the single-launch stacked step (moe_decode_step) against the
oracle's stacked step, at small shapes where every layer can be compared one to one
(inputs resampled until every routing decision and argmax has an oracle margin of at
least 1e-3): expert ids, tokens and accepted lengths bit-exact, each layer's y_l
within the bf16 tolerance."""
import numpy as np
import pytest
import torch

import oracle
import synth
from fine_grained_moe_router_amd import native
from fine_grained_moe_router_amd.stack import FusedDecodeStep
from parity_util import bf16_f64, check_bf16_output, rel_l2, stack_decisions_unambiguous, to_device

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def make(shape, seed=0, expert_dtype="fp8", router_bias=None, lm_bf16=False, router_dtype="bf16"):
    layers = [synth.layer_weights(shape, l, "cpu", seed=seed, tag="fused", expert_dtype=expert_dtype,
                                  router_bias=router_bias, router_dtype=router_dtype) for l in range(shape.layers)]
    host = [synth.weights_to_host(w) for w in layers]
    gains = synth.rmsnorm_gains(shape, seed=seed)
    if lm_bf16:   # the BF16 lm_head rung: bf16 weights, no scales (s stays None)
        Q, s = synth.lm_head_bf16(shape, seed=seed), None
    else:
        Q, s = synth.lm_head(shape, seed=seed)
    dev = [to_device(w) for w in layers]
    return layers, host, gains, Q, s, dev


def oracle_step(shape, host, gains, Q, s, M, step):
    lm_bf16 = Q.dtype == torch.bfloat16
    for sub in range(60):
        x = synth.hidden_inputs(shape, M, step, sub)
        noise = synth.stack_noise(shape, M, step, sub)
        res = oracle.stack_step(synth.bits16(x), host, synth.bits16(noise), synth.bits16(gains),
                                synth.bits16(Q) if lm_bf16 else synth.bytes8(Q), None if lm_bf16 else synth.f32(s),
                                shape.top_k, lm_bf16=lm_bf16)
        if stack_decisions_unambiguous(res):
            return x, noise, res
    raise RuntimeError("no unambiguous input")


def run_and_check(shape, M, step, seed=0, what="", expert_dtype="fp8", router_bias=None, cooperative=False,
                  lm_bf16=False, router_dtype="bf16"):
    layers, host, gains, Q, s, dev = make(shape, seed, expert_dtype, router_bias, lm_bf16, router_dtype)
    x, noise, res = oracle_step(shape, host, gains, Q, s, M, step)
    drafts = synth.drafts(res["tok"], 0.7, shape.vocab, step)
    n_ref, out_ref = oracle.spec_accept(drafts, res["tok"])
    fs = FusedDecodeStep(shape, dev, gains.to(DEV), Q.to(DEV), None if s is None else s.to(DEV), max_M=8,
                         cooperative=cooperative)
    dd = torch.from_numpy(drafts.astype(np.int32)).to(DEV) if M > 1 else None
    fs.step(x.to(DEV), noise.to(DEV), dd, M)
    torch.cuda.synchronize()
    assert fs.status() == native.MOE_OK
    idx, y = fs.topk_idx(M).cpu().numpy(), fs.y(M)
    for l in range(shape.layers):
        r = res["layers"][l]
        assert (idx[l] == r["idx"]).all(), "%s layer %d expert ids differ" % (what, l)
        # the step computes each layer's normalised input u itself: one-ulp bf16 differences
        # from the oracle's u (and, past layer 0, the drift of the two residual streams)
        # move the logits by ~1e-4, hence a looser bound on the routing weights than when u
        # is given
        np.testing.assert_allclose(fs.topk_w(M)[l].cpu().numpy(), r["w"], rtol=2e-3, atol=1e-5)
        check_bf16_output(synth.bits16(y[l]), r["y"], None, "%s y layer %d" % (what, l))
    xf = synth.bits16(fs.x_final[:M])
    assert rel_l2(bf16_f64(xf), bf16_f64(res["x_final"])) <= 2e-3, "%s x_final" % what
    assert (xf == res["x_final"]).mean() > 0.95, "%s x_final" % what
    assert (fs.tok[:M].cpu().numpy() == res["tok"]).all(), what
    np.testing.assert_allclose(fs.max_logit[:M].cpu().numpy(), res["max_logit"], rtol=2e-3, atol=1e-4)
    assert int(fs.accepted[0]) == n_ref and (fs.out_tokens[:M].cpu().numpy() == out_ref).all(), what
    return fs, x, noise, dd


@pytest.mark.parametrize("router_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("M", [1, 5])
def test_fused_step_expert_major_router(router_dtype, M):
    """MOE_ROUTER_EXPERT_MAJOR in the fused step: prepare copies the [E][H] routers as they
    are instead of transposing them, and the step is bit-identical to the [H][E] one."""
    sh = synth.TINY.with_(layers=2)
    layers, host, gains, Q, s, dev = make(sh, 4, "fp8", None, False, router_dtype)
    x, noise, res = oracle_step(sh, host, gains, Q, s, M, 40 + M)
    drafts = synth.drafts(res["tok"], 0.7, sh.vocab, 40 + M)
    dd = torch.from_numpy(drafts.astype(np.int32)).to(DEV) if M > 1 else None
    a = FusedDecodeStep(sh, dev, gains.to(DEV), Q.to(DEV), s.to(DEV), max_M=8)
    em = [dict(w, router_w=w["router_w"].t().contiguous()) for w in dev]
    b = FusedDecodeStep(sh, em, gains.to(DEV), Q.to(DEV), s.to(DEV), max_M=8)
    b.desc.layer.router_type |= native.MOE_ROUTER_EXPERT_MAJOR
    native.moe_decode_step_prepare(b.desc, [native.layer_weights(w) for w in em], b.ws, b.ws_bytes)
    for f in (a, b):
        f.step(x.to(DEV), noise.to(DEV), dd, M)
    torch.cuda.synchronize()
    assert a.status() == native.MOE_OK and b.status() == native.MOE_OK
    assert (a.topk_idx(M).cpu() == b.topk_idx(M).cpu()).all()
    assert (a.topk_w(M).cpu() == b.topk_w(M).cpu()).all()
    assert (synth.bits16(a.y(M)) == synth.bits16(b.y(M))).all()
    assert (a.tok[:M].cpu() == b.tok[:M].cpu()).all() and (a.tok[:M].cpu().numpy() == res["tok"]).all()


@pytest.mark.parametrize("L", [1, 2, 3])
@pytest.mark.parametrize("M", [1, 5, 8])
def test_fused_step_tiny(L, M):
    say("fused tiny L=%d M=%d" % (L, M))
    run_and_check(synth.TINY.with_(layers=L), M, step=10 * L + M, what="L=%d M=%d" % (L, M))


@pytest.mark.parametrize("experts", ["fp8", "bf16"])
@pytest.mark.parametrize("M", [1, 5, 8])
def test_fused_step_bf16_lm_head(M, experts):
    """The precision ladder's BF16 rungs: a bf16 lm_head (no scales), with FP8 or bf16 experts."""
    say("fused bf16 lm_head M=%d experts %s" % (M, experts))
    run_and_check(FUSED_VARIANTS["h2816"], M, step=70 + M, seed=8, what="bf16 lm_head M=%d" % M,
                  expert_dtype=experts, lm_bf16=True)


@pytest.mark.parametrize("name", ["tiny", "e48_k6", "h2816"])
@pytest.mark.parametrize("M", [1, 5, 8])
def test_fused_step_fp8_router(name, M):
    """The precision ladder's FP8 router rung in the fused step: codes re-laid out one expert
    per row at prepare, widened to bf16 in the router workgroups, the expert's scale applied to
    the finished logit."""
    sh = synth.TINY.with_(layers=2) if name == "tiny" else FUSED_VARIANTS[name]
    say("fused fp8 router %s M=%d" % (name, M))
    run_and_check(sh, M, step=90 + M, seed=9, what="fp8 router %s M=%d" % (name, M), router_dtype="fp8")


@pytest.mark.parametrize("M", [1, 5, 8])
def test_fused_step_cooperative_launch(M):
    """The opt-in cooperative launch (every workgroup resident before any starts) gives
    the same results as the oracle."""
    say("fused cooperative M=%d" % M)
    run_and_check(synth.TINY.with_(layers=2), M, step=30 + M, what="coop M=%d" % M, cooperative=True)


FUSED_VARIANTS = {
    "no_shared": synth.TINY.with_(shared_width=0, layers=2),
    "wide_shared": synth.TINY.with_(shared_width=192, layers=2),
    "e256_k8": synth.TINY.with_(experts=256, top_k=8, hidden=512, width=128, shared_width=64, layers=2),
    "e128_k16": synth.TINY.with_(experts=128, top_k=16, hidden=768, layers=2),
    "e48_k6": synth.TINY.with_(experts=48, top_k=6, layers=2),
    "h2816": synth.TINY.with_(hidden=2816, experts=32, top_k=4, width=704, shared_width=704, vocab=8192,
                              layers=2),
    # the page's 2112-wide always-on MLP as the shared expert: three 704-column down segments
    "h2816_sh2112": synth.TINY.with_(hidden=2816, experts=32, top_k=4, width=704, shared_width=2112,
                                     vocab=8192, layers=2),
}


@pytest.mark.parametrize("name", sorted(FUSED_VARIANTS))
@pytest.mark.parametrize("M", [1, 8])
def test_fused_step_variants(name, M):
    say("fused variant %s M=%d" % (name, M))
    run_and_check(FUSED_VARIANTS[name], M, step=500 + M, seed=2, what=name)


@pytest.mark.parametrize("name", ["tiny", "h2816"])
@pytest.mark.parametrize("M", [1, 5, 8])
def test_fused_step_bf16_experts(name, M):
    """bf16 expert weights: half the rows per unit, the same hand-offs."""
    sh = synth.TINY.with_(layers=2) if name == "tiny" else FUSED_VARIANTS["h2816"]
    say("fused bf16 %s M=%d" % (name, M))
    run_and_check(sh, M, step=600 + M, seed=5, what="bf16 " + name, expert_dtype="bf16")


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_fused_step_zipf_router_bias_m8(dtype):
    """The skewed-routing configuration in small: M=8 with a Zipf router bias."""
    sh = synth.TINY.with_(experts=64, top_k=4, hidden=512, width=128, layers=2)
    say("fused zipf M=8 %s" % dtype)
    run_and_check(sh, 8, step=700, seed=6, what="zipf " + dtype, expert_dtype=dtype,
                  router_bias=synth.zipf_router_bias(64))


@pytest.mark.parametrize("M", [1, 5, 8])
def test_fused_step_routing_ties_go_to_lower_id(M):
    """Exact ties among the router logits: with zero router weights and a bias that gives
    six experts the same largest logit, every token of every layer selects the K lowest
    ids of the six, each with weight exactly 1/K (at M=5 and M=8 a wave selects two
    tokens in the same rounds), and the layer outputs match the oracle's, which breaks
    ties the same way."""
    sh = synth.TINY.with_(experts=64, top_k=4, hidden=512, width=128, layers=2)
    tied = [3, 7, 9, 12, 40, 50]
    bias = torch.zeros(64, dtype=torch.float32)
    bias[tied] = 1.0
    layers, host, gains, Q, s, dev = make(sh, seed=9, router_bias=bias)
    for w, hw in zip(dev, host):
        w["router_w"] = torch.zeros_like(w["router_w"])
        hw["router_w"] = np.zeros_like(hw["router_w"])
    x = synth.hidden_inputs(sh, M, 0, 0)
    noise = synth.stack_noise(sh, M, 0, 0)
    res = oracle.stack_step(synth.bits16(x), host, synth.bits16(noise), synth.bits16(gains),
                            synth.bytes8(Q), synth.f32(s), sh.top_k)
    say("fused routing ties M=%d" % M)
    fs = FusedDecodeStep(sh, dev, gains.to(DEV), Q.to(DEV), s.to(DEV), max_M=8)
    dd = torch.zeros(M - 1, dtype=torch.int32, device=DEV) if M > 1 else None
    fs.step(x.to(DEV), noise.to(DEV), dd, M)
    torch.cuda.synchronize()
    assert fs.status() == native.MOE_OK
    want = np.array(tied[:sh.top_k])
    idx, wts, y = fs.topk_idx(M).cpu().numpy(), fs.topk_w(M).cpu().numpy(), fs.y(M)
    assert (idx == want).all(), idx
    assert (wts == np.float32(1.0 / sh.top_k)).all(), wts
    for l in range(sh.layers):
        assert (res["layers"][l]["idx"] == want).all()
        check_bf16_output(synth.bits16(y[l]), res["layers"][l]["y"], None, "ties y layer %d" % l)


def test_fused_step_batch_consistency_and_determinism():
    sh = synth.TINY.with_(experts=64, top_k=4, hidden=512, width=128, layers=3)
    layers, host, gains, Q, s, dev = make(sh, seed=3)
    fs = FusedDecodeStep(sh, dev, gains.to(DEV), Q.to(DEV), s.to(DEV), max_M=8)
    x = synth.hidden_inputs(sh, 5, 0).to(DEV)
    noise = synth.stack_noise(sh, 5, 0).to(DEV)
    d = torch.zeros(4, dtype=torch.int32, device=DEV)
    fs.step(x, noise, d, 5)
    torch.cuda.synchronize()
    y5, t5, i5 = fs.y(5).clone(), fs.tok[:5].clone(), fs.topk_idx(5).clone()
    fs.step(x, noise, d, 5)
    torch.cuda.synchronize()
    assert torch.equal(fs.y(5), y5) and torch.equal(fs.tok[:5], t5)
    for m in range(5):
        fs.step(x[m:m + 1].contiguous(), noise[:, m:m + 1].contiguous(), None, 1)
        torch.cuda.synchronize()
        assert torch.equal(fs.y(1)[:, 0], y5[:, m]) and int(fs.tok[0]) == int(t5[m])
        assert torch.equal(fs.topk_idx(1)[:, 0], i5[:, m])
    assert fs.status() == native.MOE_OK


def test_fused_step_graph_capture_replays():
    sh = synth.TINY.with_(layers=3)
    layers, host, gains, Q, s, dev = make(sh, seed=4)
    fs = FusedDecodeStep(sh, dev, gains.to(DEV), Q.to(DEV), s.to(DEV), max_M=5)
    x = synth.hidden_inputs(sh, 5, 1).to(DEV)
    noise = synth.stack_noise(sh, 5, 1).to(DEV)
    d = torch.arange(4, dtype=torch.int32, device=DEV)
    fs.step(x, noise, d, 5)
    torch.cuda.synchronize()
    ref = (fs.y(5).clone(), fs.tok[:5].clone(), fs.accepted.clone())
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            fs.step(x, noise, d, 5)
    torch.cuda.current_stream().wait_stream(st)
    for rep in range(3):
        fs._y.zero_()
        fs.tok.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(fs.y(5), ref[0]) and torch.equal(fs.tok[:5], ref[1]), rep
        _ = torch.ones(512, device=DEV).sum().item()
    assert fs.status() == native.MOE_OK


def test_fused_step_timeout_then_recovers():
    """A spin limit of one poll makes the step's own bounded waits give up (no wait is
    satisfied on its first poll): every workgroup still exits, the status reports the
    timeout, and the next step on the same workspace with the default limit matches
    the oracle."""
    sh = synth.TINY.with_(layers=2)
    M = 5
    layers, host, gains, Q, s, dev = make(sh, seed=11)
    x, noise, res = oracle_step(sh, host, gains, Q, s, M, step=800)
    drafts = synth.drafts(res["tok"], 0.7, sh.vocab, 800)
    n_ref, out_ref = oracle.spec_accept(drafts, res["tok"])
    fs = FusedDecodeStep(sh, dev, gains.to(DEV), Q.to(DEV), s.to(DEV), max_M=8, spin_limit=1)
    dd = torch.from_numpy(drafts.astype(np.int32)).to(DEV)
    say("fused step with spin limit 1")
    fs.step(x.to(DEV), noise.to(DEV), dd, M)
    torch.cuda.synchronize()
    assert fs.status() == native.MOE_ETIMEOUT
    assert fs.status() == native.MOE_OK          # cleared
    fs.desc.spin_limit = 0
    say("fused step with the default spin limit")
    for rep in range(2):
        fs.step(x.to(DEV), noise.to(DEV), dd, M)
        torch.cuda.synchronize()
        assert fs.status() == native.MOE_OK
        idx, y = fs.topk_idx(M).cpu().numpy(), fs.y(M)
        for l in range(sh.layers):
            assert (idx[l] == res["layers"][l]["idx"]).all(), (rep, l)
            check_bf16_output(synth.bits16(y[l]), res["layers"][l]["y"], None, "y layer %d" % l)
        assert (fs.tok[:M].cpu().numpy() == res["tok"]).all()
        assert int(fs.accepted[0]) == n_ref and (fs.out_tokens[:M].cpu().numpy() == out_ref).all()
