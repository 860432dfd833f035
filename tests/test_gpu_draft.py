"""GPU parity of the MTP drafter step (moe_draft_step) against the oracle's drafter step:
gamma drafts in sequence, each chaining on the previous one on the device. The starting
token and hidden state are resampled until every draft's argmax has an oracle margin of
at least TAU; then the drafted tokens must match bit for bit. Heads that fit it run the
one-launch (persistent) form by default; `chain=True` forces the chain of launches, so
both forms are checked at the same shapes."""
import numpy as np
import pytest
import torch

import oracle
import synth
from fine_grained_moe_router_amd import native

pytestmark = pytest.mark.gpu
DEV = "cuda"
# The oracle rounds each stage's fp64 sums to bf16; the kernels round fp32 sums taken in
# another order. Where a value lies that close to a bf16 rounding boundary the two round
# apart by one bf16 step (2^-8 relative), and that difference travels through the later
# blocks and drafts. A margin of 1e-3 was not enough for four drafts of the small head (a
# third-draft margin of 1.65e-3 flipped in both the chain and the one-launch form, which
# agree with each other bit for bit there); 1e-2 leaves six times that headroom.
TAU = 1e-2
TINY_TARGET = synth.TINY.with_(vocab=synth.TINY_HEAD.vocab)


def say(*a):
    print(*a, flush=True)


class Case:
    """A head, the target's tied table and one unambiguous drafter input (tok0, g0) with
    the oracle's drafts."""

    def __init__(self, head_shape, target_shape, seed, gamma=4, device_gen="cpu", sub0=0):
        self.shape, self.gamma = head_shape, gamma
        w = synth.draft_head(head_shape, device_gen, seed=seed)
        host = synth.draft_head_to_host(w, head_shape)
        Qt, st = synth.lm_head(target_shape, device_gen, seed=seed)
        Qh, sh = synth.bytes8(Qt), synth.f32(st)
        for sub in range(sub0, sub0 + 30):
            g0 = synth.hidden_inputs(target_shape, 1, sub, tag="draft_g")
            tok0 = (sub * 7919 + 11) % target_shape.vocab
            r = oracle.draft_step(tok0, synth.bits16(g0)[0], host, Qh, sh, gamma)
            if (r["gaps"] >= TAU).all():
                break
        else:
            raise RuntimeError("no unambiguous drafter input")
        self.ref = r
        self.wd = {k: v.to(DEV) for k, v in w.items()}
        self.Qt, self.st = Qt.to(DEV), st.to(DEV)
        self.g0 = g0[0].contiguous().to(DEV)
        self.t0 = torch.tensor([tok0], dtype=torch.int32, device=DEV)

    def run(self, desc, ws, wsb, drafts=None):
        if drafts is None:
            drafts = torch.full((self.gamma,), -1, dtype=torch.int32, device=DEV)
        native.moe_draft_step(desc, native.draft_weights(self.wd), self.gamma, self.t0, self.g0, self.Qt, self.st,
                              drafts, ws, wsb)
        return drafts


def run_case(head_shape, target_shape, seed, gamma=4, device_gen="cpu", chain=False):
    c = Case(head_shape, target_shape, seed, gamma, device_gen)
    desc = native.draft_desc(head_shape, chain=chain)
    wsb = native.moe_draft_step_workspace(desc)
    ws = native.workspace(wsb)
    d = c.run(desc, ws, wsb)
    torch.cuda.synchronize()
    assert native.moe_draft_step_status(desc, ws) == native.MOE_OK
    return d.cpu().numpy(), c.ref


@pytest.mark.parametrize("chain", [False, True], ids=["fused", "chain"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_draft_step_tiny(seed, chain):
    d, r = run_case(synth.TINY_HEAD, TINY_TARGET, seed, chain=chain)
    assert (d == r["drafts"]).all(), (d, r["drafts"])


@pytest.mark.parametrize("gamma", [1, 2, 7])
def test_draft_step_tiny_gamma(gamma):
    """One draft (no post-projection), two, and the most a verify step takes."""
    d, r = run_case(synth.TINY_HEAD, TINY_TARGET, 4, gamma=gamma)
    assert (d == r["drafts"]).all(), (d, r["drafts"])


@pytest.mark.parametrize("chain", [False, True], ids=["fused", "chain"])
def test_draft_step_no_blocks(chain):
    """A head without body blocks: the pre-projection feeds the final norm directly."""
    hs = synth.TINY_HEAD.__class__(hidden=256, width=256, ffn=512, blocks=0, vocab=1024)
    d, r = run_case(hs, TINY_TARGET, 6, chain=chain)
    assert (d == r["drafts"]).all(), (d, r["drafts"])


# Shapes that make each kernel of the chain read its rows with 16, 32 and 64 lanes per row
# somewhere in the set (pre_projection, gate/up, down, post-projection): the full-size head
# takes 32/16/64/32 and TINY_HEAD 32/16/32/16 there; the first two here are wider than the
# one-launch form takes and run the chain (32/64/32/64 and 16/32/16/64). The others run the
# one-launch form, whose lanes per row (pre, gate/up, down, post) are 128/32/32/32 for the
# full-size head and 128/256/16/128 for TINY_HEAD: 128/16/64/128 (64 down workgroups of
# four rows), 128/64/16/128 (two blocks), 128/32/32/128 (a 768-wide head: three 256-column
# table chunks, 384 pre-projection workgroups) and 128/16/64/128 with an inner width of 6144.
SPLIT_SHAPES = [synth.DraftShape(hidden=512, width=2048, ffn=1024, blocks=1, vocab=2048),    # 32/64/32/64
                synth.DraftShape(hidden=256, width=4096, ffn=2048, blocks=1, vocab=1024),    # 16/32/16/64
                synth.DraftShape(hidden=1024, width=256, ffn=8192, blocks=1, vocab=1024),
                synth.DraftShape(hidden=512, width=512, ffn=2048, blocks=2, vocab=2048),
                synth.DraftShape(hidden=1024, width=768, ffn=3072, blocks=1, vocab=1024),
                synth.DraftShape(hidden=512, width=256, ffn=6144, blocks=1, vocab=1024)]


@pytest.mark.parametrize("hs", SPLIT_SHAPES, ids=lambda h: "h%d_w%d_f%d" % (h.hidden, h.width, h.ffn))
def test_draft_step_row_splits(hs):
    say("drafter %s" % (hs,))
    d, r = run_case(hs, synth.TINY.with_(hidden=hs.hidden, vocab=hs.vocab), 7)
    assert (d == r["drafts"]).all(), (d, r["drafts"])


@pytest.mark.parametrize("chain", [False, True], ids=["fused", "chain"])
def test_draft_step_mtp_head_full_size(chain):
    """The 430M head at the Gemma-4-26B-A4B shape: 2816-wide target, 1024-wide head, 12 blocks,
    262,144-row tables."""
    say("drafter, full size, chain=%s" % chain)
    d, r = run_case(synth.MTP_HEAD, synth.GEMMA4_26B_A4B, 3, device_gen=DEV, chain=chain)
    say("drafts %s (oracle %s), margins %s" % (list(d), list(r["drafts"]), np.round(r["gaps"], 4)))
    assert (d == r["drafts"]).all()


@pytest.mark.parametrize("chain", [False, True], ids=["fused", "chain"])
def test_draft_step_is_deterministic(chain):
    a, _ = run_case(synth.TINY_HEAD, TINY_TARGET, 5, chain=chain)
    b, _ = run_case(synth.TINY_HEAD, TINY_TARGET, 5, chain=chain)
    assert (a == b).all()


def test_draft_step_workspace_reuse():
    """Calls on one workspace advance its call counter: two inputs alternated four times,
    every call's drafts as the oracle's."""
    c1 = Case(synth.TINY_HEAD, TINY_TARGET, 8, sub0=0)
    c2 = Case(synth.TINY_HEAD, TINY_TARGET, 9, sub0=40)
    desc = native.draft_desc(synth.TINY_HEAD)
    wsb = native.moe_draft_step_workspace(desc)
    ws = native.workspace(wsb)
    for rep in range(4):
        for c in (c1, c2):
            d = c.run(desc, ws, wsb)
            torch.cuda.synchronize()
            assert (d.cpu().numpy() == c.ref["drafts"]).all(), rep
    assert native.moe_draft_step_status(desc, ws) == native.MOE_OK


def test_draft_step_graph_replay():
    """The one-launch form captured in a HIP graph: each replay (with eager work between
    them) gives the oracle's drafts."""
    c = Case(synth.TINY_HEAD, TINY_TARGET, 10)
    desc = native.draft_desc(synth.TINY_HEAD)
    wsb = native.moe_draft_step_workspace(desc)
    ws = native.workspace(wsb)
    drafts = torch.full((c.gamma,), -1, dtype=torch.int32, device=DEV)
    c.run(desc, ws, wsb, drafts)   # warm-up, outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g.capture_begin()
        native.moe_draft_step(desc, native.draft_weights(c.wd), c.gamma, c.t0, c.g0, c.Qt, c.st, drafts, ws, wsb,
                              stream=s.cuda_stream)
        g.capture_end()
    torch.cuda.synchronize()
    for rep in range(3):
        drafts.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert (drafts.cpu().numpy() == c.ref["drafts"]).all(), rep
        _ = torch.ones(512, device=DEV).sum().item()
    assert native.moe_draft_step_status(desc, ws) == native.MOE_OK


def test_draft_step_timeout_then_recovers():
    """A spin limit of one poll makes the one-launch form's bounded waits give up (no wait is
    satisfied on its first poll): every workgroup still exits, the status reports the
    timeout once, and the next calls on the same workspace with the default limit give the
    oracle's drafts."""
    c = Case(synth.TINY_HEAD, TINY_TARGET, 11)
    desc = native.draft_desc(synth.TINY_HEAD, spin_limit=1)
    wsb = native.moe_draft_step_workspace(desc)
    ws = native.workspace(wsb)
    say("drafter with spin limit 1")
    c.run(desc, ws, wsb)
    torch.cuda.synchronize()
    assert native.moe_draft_step_status(desc, ws) == native.MOE_ETIMEOUT
    assert native.moe_draft_step_status(desc, ws) == native.MOE_OK   # cleared
    desc.spin_limit = 0
    say("drafter with the default spin limit")
    for rep in range(2):
        d = c.run(desc, ws, wsb)
        torch.cuda.synchronize()
        assert native.moe_draft_step_status(desc, ws) == native.MOE_OK
        assert (d.cpu().numpy() == c.ref["drafts"]).all(), rep
