"""Pins of the oracle's greedy acceptance (CPU only).

* brute force over every draft/target pair on a two-letter alphabet, against
  the definition "number of leading positions where draft == target", computed
  independently as a cumulative product;
* closed form: with independent agreement probabilities p_d per depth, the
  expected accepted length is sum_{j=1..K} prod_{d<j} p_d; a Monte Carlo run of
  the oracle over the synthetic target generator matches it.
"""

import itertools

import numpy as np
import pytest

import oracle
import synth


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_accept_brute_force(K):
    seqs = list(itertools.product([0, 1], repeat=K))
    tgts = list(itertools.product([0, 1], repeat=K + 1))
    d = np.array([s for s in seqs for _ in tgts])
    t = np.array([s for _ in seqs for s in tgts])
    acc, bonus = oracle.accept(d, t)
    ref = np.cumprod(d == t[:, :K], axis=1).sum(axis=1)
    assert np.array_equal(acc, ref)
    assert np.array_equal(bonus, t[np.arange(len(t)), ref])


def _closed_form(p):
    return float(sum(np.prod(p[:j]) for j in range(1, len(p) + 1)))


@pytest.mark.parametrize("name", ["tiny-fp32-c2-k3", "qwen3coder30b-bf16-c16-k3",
                                  "qwen3coder30b-bf16-c16-k5", "qwen3coder30b-bf16-c16-k7"])
def test_accept_monte_carlo_matches_closed_form(name):
    wl = synth.WORKLOADS[name]
    p = wl.agree_probs()
    rounds = 20000
    rng = np.random.default_rng(5)
    drafts = rng.integers(0, wl.model.vocab, size=(rounds, wl.K))
    u = rng.random((rounds, wl.K))
    alt = rng.integers(0, wl.model.vocab - 2, size=(rounds, wl.K + 1))
    tgt = synth.target_tokens_from_drafts(drafts, u, alt, p, wl.model.vocab)
    acc, _ = oracle.accept(drafts, tgt)
    expect = _closed_form(p)
    se = acc.std() / np.sqrt(rounds)
    assert abs(acc.mean() - expect) < 5 * se + 1e-9


def test_closed_form_values():
    # agreement 0.8 * 0.9^d per depth
    for K, v in [(3, 1.7488), (5, 2.0813), (7, 2.1584)]:
        p = 0.8 * 0.9 ** np.arange(K)
        assert abs(_closed_form(p) - v) < 1e-3
