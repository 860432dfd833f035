"""Pins of the oracle's stochastic speculative acceptance (no GPU).

The page says a drafted token is kept only if it passes the exact distribution the
target would have sampled from, so that the output is distributed as ordinary
decoding (page "LLM decoding", "What we learned, and where this goes"). The oracle
takes the standard rule (accept with probability min(1, p/q), else draw from the
normalised residual max(0, p - q), or the bonus token from p), drawing with the
Gumbel-max rule over Philox4x32-10 uniforms. Pinned here against:
  * the generator's published known-answer vectors,
  * the accept region's closed form, exhaustively on a tiny vocabulary,
  * the Gumbel-max rule's distribution (chi-square over many counters),
  * the exactness property itself: the emitted tokens are distributed as p
    (chi-square), with planted mistakes in a numpy copy of the rule rejected by the
    same test.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answer_vectors():
    kat = json.load(open(os.path.join(GOLDEN, "philox4x32_10_kat.json")))
    for v in kat["vectors"]:
        ctr = [int(w, 16) for w in v["ctr"]]
        key = [int(w, 16) for w in v["key"]]
        out = oracle.philox4x32_10(ctr, key)
        assert ["%08x" % w for w in out] == v["out"]


def test_sample_uniform_uses_the_documented_counter():
    # (v / 4, row, step low, step high) under key (seed low, seed high), word v % 4, (x + 1/2) / 2^32
    seed, step = 0x0123456789ABCDEF, 0x1122334455667788
    for row, v in ((0, 0), (3, 5), (4, 262143)):
        w = oracle.philox4x32_10([v >> 2, row, step & 0xFFFFFFFF, step >> 32],
                                 [seed & 0xFFFFFFFF, seed >> 32])[v & 3]
        assert oracle.sample_uniform(seed, step, row, v) == (float(w) + 0.5) / 2.0 ** 32


def softmax(z):
    z = np.asarray(z, np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


def test_accept_region_is_min_one_p_over_q():
    """For every draft id of a tiny vocabulary, the fraction of a uniform grid of u that
    accepts equals min(1, p(d) / q(d)) to the grid's resolution."""
    V, T = 5, 0.7
    rng = np.random.default_rng(0)
    logits = rng.normal(size=(2, V))
    q = softmax(rng.normal(size=V)).astype(np.float32)[None, :]
    p0 = softmax(logits[0] / T)
    grid = (np.arange(2000) + 0.5) / 2000
    for d in range(V):
        acc = 0
        for u in grid:
            n, out, _, _ = oracle.spec_sample(logits, T, np.array([d], np.int32), q, np.array([u], np.float32),
                                              seed=1, step=2)
            acc += n
        assert abs(acc / len(grid) - min(1.0, p0[d] / float(q[0, d]))) <= 1.0 / len(grid) + 1e-3, d


def test_out_of_range_drafts_are_rejected():
    V, T = 4, 1.0
    logits = np.zeros((2, V))
    q = np.full((1, V), 0.25, np.float32)
    for d in (-1, V, 1 << 30):
        n, out, am, _ = oracle.spec_sample(logits, T, np.array([d], np.int32), q, np.array([0.0], np.float32), 0, 0)
        assert n == 0 and out[1] == -1 and 0 <= out[0] < V and am[0] == math.inf


def _chi2_ok(counts, probs, alpha=1e-4):
    counts = np.asarray(counts, np.float64)
    exp = probs * counts.sum()
    keep = exp > 0
    assert counts[~keep].sum() == 0, "draws where the distribution is zero"
    stat = ((counts[keep] - exp[keep]) ** 2 / exp[keep]).sum()
    return stats.chi2.sf(stat, keep.sum() - 1) > alpha


def test_gumbel_max_draws_follow_the_bonus_distribution():
    """All drafts accepted (q = p, u = 0): the last token is the bonus draw from p_gamma,
    which the Gumbel-max rule over the uniforms makes exact; frequencies over 20,000
    counters follow p (chi-square)."""
    V, T, N = 6, 0.7, 20000
    rng = np.random.default_rng(1)
    logits = rng.normal(size=(2, V)) * 1.5
    p1 = softmax(logits[1] / T)
    q = softmax(logits[0] / T).astype(np.float32)[None, :]
    counts = np.zeros(V)
    for step in range(N):
        n, out, _, _ = oracle.spec_sample(logits, T, np.array([0], np.int32), q, np.array([0.0], np.float32),
                                          seed=7, step=step)
        assert n == 1 and out[0] == 0
        counts[out[1]] += 1
    assert _chi2_ok(counts, p1)


def _emitted_distribution_trial(sampler, logits, T, q, rng, trials, seed):
    """Run the rule `trials` times with drafts d_i ~ q_i and fresh uniforms; count the
    token emitted at positions 0 and 1 (position 1 when it exists)."""
    M, V = logits.shape
    c0, c1 = np.zeros(V), np.zeros(V)
    for t in range(trials):
        d = np.array([rng.choice(V, p=q[i] / q[i].sum()) for i in range(M - 1)], np.int32)
        u = rng.random(M - 1).astype(np.float32)
        n, out = sampler(logits, T, d, q, u, seed, t)
        c0[out[0]] += 1
        if n >= 1:
            c1[out[1]] += 1
    return c0, c1


def _oracle_sampler(logits, T, d, q, u, seed, step):
    n, out, _, _ = oracle.spec_sample(logits, T, d, q, u, seed, step)
    return n, out


@pytest.mark.parametrize("gamma", [1, 2])
def test_emitted_tokens_are_distributed_as_the_target(gamma):
    """The exactness property: with drafts drawn from q, the emitted token at position 0
    follows p_0 and, where it exists, the one at position 1 follows p_1."""
    V, T, N = 6, 0.7, 20000
    rng = np.random.default_rng(10 + gamma)
    logits = rng.normal(size=(gamma + 1, V)) * 1.5
    q = np.stack([softmax(rng.normal(size=V) * 1.5) for _ in range(gamma)]).astype(np.float32)
    c0, c1 = _emitted_distribution_trial(_oracle_sampler, logits, T, q, rng, N, seed=3)
    assert _chi2_ok(c0, softmax(logits[0] / T))
    assert _chi2_ok(c1, softmax(logits[1] / T))
    assert 0.2 * N < c1.sum() < 0.95 * N      # the drafts are neither always nor never accepted


def _planted_sampler(kind):
    """A numpy copy of the rule with one plausible mistake."""
    def sampler(logits, T, d, q, u, seed, step):
        M, V = logits.shape
        p = np.stack([softmax(l / T) for l in logits])
        n = 0
        while n < M - 1:
            ratio = p[n, d[n]] / q[n, d[n]]
            if kind == "accept_on_q_over_p":
                ratio = q[n, d[n]] / p[n, d[n]]
            if not (u[n] < ratio):
                break
            n += 1
        if n < M - 1:
            r = np.maximum(0.0, p[n] - q[n])
            if kind == "resample_from_p":
                r = p[n]
            if kind == "residual_wrong_row":
                r = np.maximum(0.0, p[n] - q[(n + 1) % (M - 1)])
        else:
            r = p[n]
        g = np.array([-math.log(-math.log(oracle.sample_uniform(seed, step, n, v))) for v in range(V)])
        with np.errstate(divide="ignore"):
            t = int(np.argmax(np.where(r > 0, np.log(r) + g, -np.inf)))
        out = np.full(M, -1, np.int32)
        out[:n] = d[:n]
        out[n] = t
        return n, out
    return sampler


@pytest.mark.parametrize("kind", ["accept_on_q_over_p", "resample_from_p", "residual_wrong_row"])
def test_exactness_test_rejects_planted_mistakes(kind):
    V, T, N = 6, 0.7, 8000
    rng = np.random.default_rng(20)
    gamma = 2
    logits = rng.normal(size=(gamma + 1, V)) * 1.5
    q = np.stack([softmax(rng.normal(size=V) * 1.5) for _ in range(gamma)]).astype(np.float32)
    c0, c1 = _emitted_distribution_trial(_planted_sampler(kind), logits, T, q, rng, N, seed=4)
    assert not (_chi2_ok(c0, softmax(logits[0] / T)) and _chi2_ok(c1, softmax(logits[1] / T))), kind


def test_correct_numpy_copy_passes_the_same_test():
    V, T, N = 6, 0.7, 8000
    rng = np.random.default_rng(20)
    gamma = 2
    logits = rng.normal(size=(gamma + 1, V)) * 1.5
    q = np.stack([softmax(rng.normal(size=V) * 1.5) for _ in range(gamma)]).astype(np.float32)
    c0, c1 = _emitted_distribution_trial(_planted_sampler("none"), logits, T, q, rng, N, seed=4)
    assert _chi2_ok(c0, softmax(logits[0] / T)) and _chi2_ok(c1, softmax(logits[1] / T))


def test_lm_head_logits_match_the_argmax_routine():
    import synth
    sh = synth.TINY
    Q, s = synth.lm_head(sh, seed=2)
    x = synth.bits16(synth.hidden_inputs(sh, 3, 0))
    lg = oracle.lm_head_logits(x, synth.bytes8(Q), synth.f32(s))
    tok, ml, _ = oracle.lm_head_argmax(x, synth.bytes8(Q), synth.f32(s))
    assert (lg.argmax(axis=1) == tok).all() and np.allclose(lg.max(axis=1), ml, rtol=0, atol=0)
    rows = np.array([0, 17, 4095], np.int32)
    assert np.array_equal(oracle.lm_head_rows(x, synth.bytes8(Q), synth.f32(s), rows), lg[:, rows])
