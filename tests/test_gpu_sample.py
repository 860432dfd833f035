"""GPU parity of lm_head_spec_sample (stochastic speculative acceptance at temperature
0.7 on the tied lm_head) against the oracle.

The drafter's distributions are synthetic: q_i is a softmax of the oracle's own target
logits for row i - 1 plus seeded Gaussian noise (at temperature T), so acceptance is
high but not certain, and no GPU value enters an input or an expected value. Drafts
d_i ~ q_i and the accept uniforms are seeded. Each case is resampled (new uniforms and a
new Philox step) until every accept decision and the final draw have an oracle margin of
at least 1e-3 (float32 logits and log-normalisers are good to about 1e-5 in these
units); then the accepted length and every emitted token must match bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from fine_grained_moe_router_amd import native

pytestmark = pytest.mark.gpu
DEV = "cuda"
T = 0.7
TAU = 1e-3


def say(*a):
    print(*a, flush=True)


def softmax(z):
    e = np.exp(z - z.max())
    return e / e.sum()


class Head:
    def __init__(self, shape, seed):
        self.shape = shape
        Q, s = synth.lm_head(shape, DEV if shape.vocab > 65536 else "cpu", seed=seed)
        self.Qh, self.sh = synth.bytes8(Q), synth.f32(s)
        self.Q, self.s = Q.to(DEV), s.to(DEV)


def make_case(head, M, case_seed, sigma=0.3, force=None, tries=60):
    sh = head.shape
    V, gamma = sh.vocab, M - 1
    x = synth.hidden_inputs(sh, M, case_seed, tag="sample_x")
    lg = oracle.lm_head_logits(synth.bits16(x), head.Qh, head.sh)
    rng = np.random.default_rng(case_seed)
    q64 = [softmax((lg[i] + sigma * rng.normal(size=V)) / T) for i in range(gamma)]
    q = np.stack(q64).astype(np.float32) if gamma else np.zeros((0, V), np.float32)
    d = np.array([rng.choice(V, p=q64[i]) for i in range(gamma)], np.int32)
    if force == "reject_first":
        # the draft the target finds least likely relative to the drafter
        p0 = softmax(lg[0] / T)
        d[0] = int(np.argmin(p0 / np.maximum(q[0], 1e-30)))
    for t in range(tries):
        u = rng.random(gamma).astype(np.float32)
        if force == "all":
            u[:] = 0.0
        step = 1000 * case_seed + t
        n, out, am, smg = oracle.spec_sample(lg, T, d, q, u, seed=case_seed, step=step)
        if (am >= TAU).all() and smg >= TAU and (force != "reject_first" or n == 0):
            return x, q, d, u, step, n, out
    raise RuntimeError("no case with every margin above %g" % TAU)


def run_gpu(head, M, x, q, d, u, seed, step):
    sh = head.shape
    wsb = native.lm_head_spec_sample_workspace(M, sh.hidden, sh.vocab)
    ws = native.workspace(wsb)
    n = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    out = torch.full((M,), -7, dtype=torch.int32, device=DEV)
    g = M - 1
    qd = torch.from_numpy(q).to(DEV) if g else None
    dd = torch.from_numpy(d).to(DEV) if g else None
    ud = torch.from_numpy(u).to(DEV) if g else None
    native.lm_head_spec_sample(M, sh.hidden, sh.vocab, x.to(DEV), head.Q, head.s, T, dd, qd, ud, seed, step,
                               n, out, ws, wsb)
    torch.cuda.synchronize()
    return int(n[0]), out.cpu().numpy()


@pytest.fixture(scope="module")
def gemma_head():
    return Head(synth.GEMMA4_26B_A4B, seed=5)


@pytest.mark.parametrize("case_seed", range(6))
def test_spec_sample_full_vocab_m5(gemma_head, case_seed):
    x, q, d, u, step, n_ref, out_ref = make_case(gemma_head, 5, 100 + case_seed)
    n, out = run_gpu(gemma_head, 5, x, q, d, u, 100 + case_seed, step)
    say("V=262144 M=5 case %d: accepted %d (oracle %d), tokens %s" % (case_seed, n, n_ref, list(out)))
    assert n == n_ref and (out == out_ref).all(), (n, out, n_ref, out_ref)


@pytest.mark.parametrize("force", ["all", "reject_first"])
def test_spec_sample_full_vocab_bonus_and_first_rejection(gemma_head, force):
    x, q, d, u, step, n_ref, out_ref = make_case(gemma_head, 5, 200 + len(force), force=force)
    assert (n_ref == 4) if force == "all" else (n_ref == 0)
    n, out = run_gpu(gemma_head, 5, x, q, d, u, 200 + len(force), step)
    say("V=262144 M=5 %s: accepted %d, tokens %s" % (force, n, list(out)))
    assert n == n_ref and (out == out_ref).all()


def test_spec_sample_full_vocab_m1(gemma_head):
    """gamma = 0: plain sampling of one token from p_0."""
    x, q, d, u, step, n_ref, out_ref = make_case(gemma_head, 1, 300)
    n, out = run_gpu(gemma_head, 1, x, q, d, u, 300, step)
    assert n == 0 and (out == out_ref).all()


@pytest.mark.parametrize("M", [2, 5, 8])
def test_spec_sample_small_vocab(M):
    head = Head(synth.TINY, seed=6)
    for c in range(4):
        x, q, d, u, step, n_ref, out_ref = make_case(head, M, 400 + 10 * M + c, sigma=0.5)
        n, out = run_gpu(head, M, x, q, d, u, 400 + 10 * M + c, step)
        assert n == n_ref and (out == out_ref).all(), (M, c, n, out, n_ref, out_ref)


def test_spec_sample_is_deterministic_and_keyed_by_step(gemma_head):
    x, q, d, u, step, n_ref, out_ref = make_case(gemma_head, 5, 500)
    a = run_gpu(gemma_head, 5, x, q, d, u, 500, step)
    b = run_gpu(gemma_head, 5, x, q, d, u, 500, step)
    assert a[0] == b[0] and (a[1] == b[1]).all()
