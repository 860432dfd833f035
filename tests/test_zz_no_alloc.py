"""lm_head_argmax_noalloc, the allocation-free variant of lm_head_argmax for callers
that cannot allocate: through the C ABI it must give exactly the results of the
workspace entry point (same kernels), on consecutive calls that share the static
scratch, the second with a smaller input than the first."""
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


def both(M, H, V, x, Q, s):
    wsb = native.lm_head_argmax_workspace(M, H, V)
    ws = native.workspace(wsb)
    t_ws = torch.full((M,), -1, dtype=torch.int32, device=DEV)
    m_ws = torch.full((M,), float("nan"), dtype=torch.float32, device=DEV)
    native.lm_head_argmax(M, H, V, x, Q, s, t_ws, m_ws, ws, wsb)
    t_na = torch.full((M,), -1, dtype=torch.int32, device=DEV)
    m_na = torch.full((M,), float("nan"), dtype=torch.float32, device=DEV)
    native.lm_head_argmax_noalloc(M, H, V, x, Q, s, t_na, m_na)
    torch.cuda.synchronize()
    return t_ws.cpu().numpy(), m_ws.cpu().numpy(), t_na.cpu().numpy(), m_na.cpu().numpy()


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    big = synth.GEMMA4_26B_A4B          # M = 8 over the full 262,144-row lm_head: the whole scratch
    small = synth.TINY                  # then M = 2 over 4,096 rows
    cases = []
    Qb, sb = synth.lm_head(big, DEV, seed=3)
    xb = synth.hidden_inputs(big, 8, 0, device=DEV, tag="noalloc")
    cases.append(("full lm_head M=8", 8, big, xb, Qb, sb))
    Qs, ss = synth.lm_head(small, seed=3)
    xs = synth.hidden_inputs(small, 2, 0, tag="noalloc")
    cases.append(("small lm_head M=2", 2, small, xs.to(DEV), Qs.to(DEV), ss.to(DEV)))
    for what, M, sh, x, Q, s in cases:
        say("noalloc vs workspace: %s" % what)
        t_ws, m_ws, t_na, m_na = both(M, sh.hidden, sh.vocab, x, Q, s)
        assert (t_na == t_ws).all(), what
        assert (m_na.view(np.uint32) == m_ws.view(np.uint32)).all(), what
        assert (t_ws >= 0).all() and (t_ws < sh.vocab).all()
    # the small case against the oracle as well (ties resolved by resampling are not needed:
    # only the tokens whose oracle margin is at least 1e-3 are compared)
    tok, ml, gap = oracle.lm_head_argmax(synth.bits16(xs), synth.bytes8(Qs), synth.f32(ss))
    sure = gap >= 1e-3
    assert (t_na[sure] == tok[sure]).all()
