"""Pins for the oracle's sampler (RWKV-Runner Albatross article, adapter
defaults and worker main loop: temperature, top-p, top-k, frequency penalty
with decay, batched sampling): special cases that reduce to argmax, the
empirical distribution against numpy's softmax, and closed forms for the
penalty counts."""
import math
from dataclasses import replace

import numpy as np
import pytest

import oracle as O
from continuous_batching_decode_forward_amd.configs import SamplingParams

PLAIN = SamplingParams(temperature=1.0, top_p=1.0, top_k=0, freq_penalty=0.0,
                       presence_penalty=0.0, penalty_decay=1.0, seed=9)


def draws(logits, sp, n=20000, counts=None):
    toks = np.empty(n, np.int64)
    for i in range(n):
        toks[i], _ = O.sample(logits, counts, sp, request_id=5, step_id=i)
    return toks


def chi2_ok(toks, probs, alpha_stat=None):
    V = len(probs)
    obs = np.bincount(toks, minlength=V).astype(np.float64)
    exp = probs * len(toks)
    keep = exp > 0
    assert np.all(obs[~keep] == 0), "sampled an id with zero probability"
    stat = ((obs[keep] - exp[keep]) ** 2 / exp[keep]).sum()
    dof = keep.sum() - 1
    # about a 1e-4 tail for these degrees of freedom
    limit = dof + 6.0 * math.sqrt(2.0 * max(dof, 1)) + 10
    return stat < limit, stat


def softmax(z):
    e = np.exp(z - z.max())
    return e / e.sum()


def test_top_k_one_and_tiny_top_p_and_zero_temperature_are_greedy():
    rng = np.random.default_rng(0)
    lg = rng.standard_normal(5000).astype(np.float32)
    best = int(np.argmax(lg))
    for sp in (replace(PLAIN, top_k=1), replace(PLAIN, top_p=1e-7),
               replace(PLAIN, temperature=0.0)):
        for step in range(20):
            tok, _ = O.sample(lg, None, sp, 1, step)
            assert tok == best


def test_unrestricted_draws_follow_softmax():
    lg = np.array([0.3, -1.0, 2.0, 0.0, 1.1, -0.2], np.float32)
    ok, stat = chi2_ok(draws(lg, PLAIN), softmax(lg.astype(np.float64)))
    assert ok, stat


def test_temperature_scales_logits():
    lg = np.array([0.3, -1.0, 2.0, 0.0, 1.1, -0.2], np.float32)
    sp = replace(PLAIN, temperature=0.5)
    ok, stat = chi2_ok(draws(lg, sp), softmax(lg.astype(np.float64) / 0.5))
    assert ok, stat


def test_top_k_keeps_the_k_largest_lowest_id_on_ties():
    lg = np.array([1.0, 3.0, 2.0, 2.0, 0.5, 2.0], np.float32)
    sp = replace(PLAIN, top_k=3)
    p = np.zeros(6)
    p[[1, 2, 3]] = softmax(lg[[1, 2, 3]].astype(np.float64))   # ids 2, 3 win the tie with 5
    ok, stat = chi2_ok(draws(lg, sp), p)
    assert ok, stat


@pytest.mark.parametrize("top_p,kept", [(0.6, [0, 1]), (0.85, [0, 1, 2]), (0.4, [0])])
def test_top_p_keeps_the_shortest_prefix_reaching_p(top_p, kept):
    probs = np.array([0.5, 0.3, 0.15, 0.05])
    lg = np.log(probs).astype(np.float32)
    sp = replace(PLAIN, top_p=top_p)
    p = np.zeros(4)
    p[kept] = probs[kept] / probs[kept].sum()
    ok, stat = chi2_ok(draws(lg, sp, n=8000), p)
    assert ok, stat


def test_draw_uses_ascending_id_cdf():
    """With a kept set {0, 1} of masses 5:3 the draw picks id 0 exactly when
    u * total < mass(0)."""
    probs = np.array([0.5, 0.3, 0.15, 0.05])
    lg = np.log(probs).astype(np.float32)
    sp = replace(PLAIN, top_p=0.6)
    for step in range(300):
        tok, info = O.sample(lg, None, sp, 5, step)
        u = O.uniform24(sp.seed, 5, step)
        assert info["u"] == u
        e0 = info["cdf_hi"] if tok == 0 else info["cdf_lo"]
        assert tok == (0 if u * info["sum_kept"] < e0 else 1)


def test_frequency_penalty_counts_closed_form_and_update_rounding():
    V = 16
    sp = replace(PLAIN, temperature=0.0, freq_penalty=0.0, penalty_decay=0.996)
    lg = np.zeros(V, np.float32)
    lg[7] = 1.0
    counts = np.zeros(V, np.float32)
    n = 50
    for step in range(n):
        before = counts.copy()
        tok, _ = O.sample(lg, counts, sp, 0, step)
        assert tok == 7
        ref = (before * np.float32(0.996)).astype(np.float32)
        ref[7] = np.float32(ref[7] + np.float32(1.0))
        assert np.array_equal(counts, ref)          # two roundings, no fused op
    closed = (1 - 0.996 ** n) / (1 - 0.996)
    assert abs(counts[7] - closed) < 1e-4 * closed
    assert np.all(np.delete(counts, 7) == 0)


def test_penalties_lower_repeated_tokens():
    V = 8
    lg = np.array([0, 0, 0, 2.0, 1.5, 0, 0, 0], np.float32)
    counts = np.zeros(V, np.float32)
    counts[3] = 1.0
    greedy = replace(PLAIN, temperature=0.0)
    assert O.sample(lg, counts.copy(), replace(greedy, freq_penalty=0.4), 0, 0)[0] == 3
    assert O.sample(lg, counts.copy(), replace(greedy, freq_penalty=0.6), 0, 0)[0] == 4
    # presence penalty: a flat cut for any id seen at least once
    c2 = np.zeros(V, np.float32)
    c2[3] = 0.01
    assert O.sample(lg, c2.copy(), replace(greedy, presence_penalty=0.6), 0, 0)[0] == 4
    assert O.sample(lg, c2.copy(), replace(greedy, presence_penalty=0.4), 0, 0)[0] == 3


def test_penalised_distribution():
    lg = np.array([0.3, -1.0, 2.0, 0.0, 1.1, -0.2], np.float32)
    counts = np.array([0, 0, 3.0, 0, 1.0, 0], np.float32)
    sp = replace(PLAIN, freq_penalty=0.5, presence_penalty=0.25, penalty_decay=1.0)
    toks = np.empty(20000, np.int64)
    for i in range(len(toks)):
        toks[i], _ = O.sample(lg, counts.copy(), sp, 3, i)
    pen = lg.astype(np.float64) - 0.5 * counts - 0.25 * (counts > 0)
    ok, stat = chi2_ok(toks, softmax(pen))
    assert ok, stat


def test_forbidden_ids_are_masked_before_the_draw():
    """Forbidden ids (the Albatross worker masks forbidden tokens before the
    penalties and the draw): forbidding the greedy pick makes temperature 0,
    top_k 1 and a tiny top_p pick the best remaining id; unrestricted draws
    follow the softmax renormalised over the allowed ids and never return a
    forbidden one."""
    rng = np.random.default_rng(3)
    lg = rng.standard_normal(3000).astype(np.float32)
    order = np.argsort(-lg.astype(np.float64), kind="stable")
    forbid = (int(order[0]), int(order[1]))
    for sp in (replace(PLAIN, top_k=1), replace(PLAIN, top_p=1e-7),
               replace(PLAIN, temperature=0.0)):
        sp = replace(sp, forbidden=forbid)
        for step in range(10):
            tok, _ = O.sample(lg, None, sp, 1, step)
            assert tok == int(order[2])
    small = np.array([0.3, -1.0, 2.0, 0.0, 1.1, -0.2], np.float32)
    sp = replace(PLAIN, forbidden=(2, 4))
    p = softmax(small.astype(np.float64))
    p[[2, 4]] = 0.0
    p /= p.sum()
    toks = draws(small, sp, n=12000)
    assert not np.isin(toks, [2, 4]).any()
    ok, stat = chi2_ok(toks, p)
    assert ok, stat
    # penalties still apply to the allowed ids, and counts still decay and
    # count the drawn token
    c = np.zeros(6, np.float32)
    c[0] = 3.0
    sp2 = replace(PLAIN, temperature=0.0, freq_penalty=10.0, penalty_decay=0.5,
                  forbidden=(2, 4))
    tok, _ = O.sample(small, c, sp2, 1, 0)
    assert tok == 3  # 0.3 - 30 for id 0; ids 2 and 4 masked; then 0.0 at id 3
    assert c[0] == np.float32(1.5) and c[3] == np.float32(1.0)
