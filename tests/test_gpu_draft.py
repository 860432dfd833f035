"""GPU parity of the MTP drafter step (moe_draft_step) against the oracle's drafter step:
gamma = 4 drafts in sequence, each chaining on the previous one on the device. The
starting token and hidden state are resampled until every draft's argmax has an oracle
margin of at least 1e-3; then the four drafted tokens must match bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
from fine_grained_moe_router_amd import native

pytestmark = pytest.mark.gpu
DEV = "cuda"
TAU = 1e-3


def say(*a):
    print(*a, flush=True)


def run_case(head_shape, target_shape, seed, gamma=4, device_gen="cpu"):
    w = synth.draft_head(head_shape, device_gen, seed=seed)
    host = synth.draft_head_to_host(w, head_shape)
    Qt, st = synth.lm_head(target_shape, device_gen, seed=seed)
    Qh, sh = synth.bytes8(Qt), synth.f32(st)
    for sub in range(30):
        g0 = synth.hidden_inputs(target_shape, 1, sub, tag="draft_g")
        tok0 = (sub * 7919 + 11) % target_shape.vocab
        r = oracle.draft_step(tok0, synth.bits16(g0)[0], host, Qh, sh, gamma)
        if (r["gaps"] >= TAU).all():
            break
    else:
        raise RuntimeError("no unambiguous drafter input")
    wd = {k: v.to(DEV) for k, v in w.items()}
    desc = native.draft_desc(head_shape)
    wsb = native.moe_draft_step_workspace(desc)
    ws = native.workspace(wsb)
    drafts = torch.full((gamma,), -1, dtype=torch.int32, device=DEV)
    t0 = torch.tensor([tok0], dtype=torch.int32, device=DEV)
    native.moe_draft_step(desc, native.draft_weights(wd), gamma, t0, g0[0].contiguous().to(DEV), Qt.to(DEV),
                          st.to(DEV), drafts, ws, wsb)
    torch.cuda.synchronize()
    return drafts.cpu().numpy(), r


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_draft_step_tiny(seed):
    d, r = run_case(synth.TINY_HEAD, synth.TINY.with_(vocab=synth.TINY_HEAD.vocab), seed)
    assert (d == r["drafts"]).all(), (d, r["drafts"])


# Shapes that make each kernel read its rows with 16, 32 and 64 lanes per row somewhere in
# the set (pre_projection, gate/up, down, post-projection): the full-size head takes
# 32/16/64/32, TINY_HEAD 32/16/32/16, and these:
SPLIT_SHAPES = [synth.DraftShape(hidden=512, width=2048, ffn=1024, blocks=1, vocab=2048),    # 32/64/32/64
                synth.DraftShape(hidden=256, width=4096, ffn=2048, blocks=1, vocab=1024),    # 16/32/16/64
                synth.DraftShape(hidden=1024, width=256, ffn=8192, blocks=1, vocab=1024)]    # 64/16/64/16


@pytest.mark.parametrize("hs", SPLIT_SHAPES, ids=lambda h: "h%d_w%d_f%d" % (h.hidden, h.width, h.ffn))
def test_draft_step_row_splits(hs):
    say("drafter %s" % (hs,))
    d, r = run_case(hs, synth.TINY.with_(hidden=hs.hidden, vocab=hs.vocab), 7)
    assert (d == r["drafts"]).all(), (d, r["drafts"])


def test_draft_step_mtp_head_full_size():
    """The 430M head at the Gemma-4-26B-A4B shape: 2816-wide target, 1024-wide head, 12 blocks,
    262,144-row tables."""
    say("drafter, full size")
    d, r = run_case(synth.MTP_HEAD, synth.GEMMA4_26B_A4B, 3, device_gen=DEV)
    say("drafts %s (oracle %s), margins %s" % (list(d), list(r["drafts"]), np.round(r["gaps"], 4)))
    assert (d == r["drafts"]).all()


def test_draft_step_is_deterministic():
    a, _ = run_case(synth.TINY_HEAD, synth.TINY.with_(vocab=synth.TINY_HEAD.vocab), 5)
    b, _ = run_case(synth.TINY_HEAD, synth.TINY.with_(vocab=synth.TINY_HEAD.vocab), 5)
    assert (a == b).all()
