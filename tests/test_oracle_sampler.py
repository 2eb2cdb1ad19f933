"""Pins of the sampler oracle: closed forms, invariants, planted scenarios and
the Gumbel-max sampling distribution."""

import json
import os

import numpy as np
import pytest
from scipy.stats import chi2 as chi2_dist

from oracle.sampler import (SamplerCfg, temperature, position_stats,
                            sampler_step, init_canvas)
from oracle.philox import renoise_id, canvas_id

HERE = os.path.dirname(os.path.abspath(__file__))


def settings():
    with open(os.path.join(HERE, "golden", "sampler_settings.json")) as f:
        return json.load(f)


def test_default_cfg_is_the_pages_settings():
    g = settings()
    c = SamplerCfg()
    assert (c.canvas_len, c.max_steps, c.temp_start, c.temp_end, c.stop_entropy) == \
        (g["canvas_len"], g["max_steps"], g["temp_start"], g["temp_end"], g["stop_entropy"])


def test_temperature_closed_form():
    expect48 = {0: 0.8, 11: 0.706383, 12: 0.697872, 23: 0.604255, 46: 0.408511, 47: 0.4}
    for s, t in expect48.items():
        assert abs(temperature(s, 48) - t) < 5e-7
    expect8 = [0.8, 0.742857, 0.685714, 0.628571, 0.571429, 0.514286, 0.457143, 0.4]
    for s, t in enumerate(expect8):
        assert abs(temperature(s, 8) - t) < 5e-7
    assert temperature(0, 1) == 0.8
    # linear: constant first difference
    d = np.diff([temperature(s, 48) for s in range(48)])
    assert np.allclose(d, -0.4 / 47, atol=1e-15)


@pytest.mark.parametrize("V", [512, 1 << 18])
def test_uniform_logits(V):
    mp, h, _ = position_stats(np.full(V, 3.25), 0.8)
    assert abs(mp - 1.0 / V) < 1e-15
    assert abs(h - np.log(V)) < 1e-9


@pytest.mark.parametrize("a,T,V,mp_ref,h_ref", [
    (12.0, 0.8, 1 << 18, 0.9257629299, 1.1906931434),
    (12.0, 0.4, 1 << 18, 0.9999999755, 7.604409e-07),
    (12.0, 0.8, 512, 0.9998437083, 0.0025006787),
    (5.0, 1.0, 512, 0.2250685432, 5.3660075705),
])
def test_two_level_closed_form(a, T, V, mp_ref, h_ref):
    """One logit a above V - 1 zeros: W = e^(a/T) + V - 1,
    maxprob = e^(a/T) / W, H = ln W - maxprob * a / T."""
    x = np.zeros(V)
    x[V // 3] = a
    mp, h, _ = position_stats(x, T)
    W = np.exp(a / T) + V - 1
    assert abs(mp - np.exp(a / T) / W) < 1e-12
    assert abs(h - (np.log(W) - (np.exp(a / T) / W) * a / T)) < 1e-9
    assert abs(mp - mp_ref) < 1e-9
    assert abs(h - h_ref) < max(1e-9, 1e-6 * h_ref)


def test_entropy_invariants():
    rng = np.random.default_rng(0)
    for _ in range(20):
        V = int(rng.integers(2, 3000))
        x = rng.standard_normal(V) * rng.uniform(0.1, 20)
        T = rng.uniform(0.3, 1.0)
        mp, h, _ = position_stats(x, T)
        assert -1e-12 <= h <= np.log(V) + 1e-12
        assert h >= -np.log(mp) - 1e-12           # Shannon >= min-entropy
        # two-pass (explicit probabilities) equals the one-pass form
        p = np.exp(x / T - (x / T).max())
        p /= p.sum()
        assert abs(h - (-(p * np.log(np.where(p > 0, p, 1))).sum())) < 1e-9
        assert abs(mp - p.max()) < 1e-15


def _one_step(logits, step, cfg, **kw):
    B, L, _ = logits.shape
    P = kw.pop("P", np.zeros(B, np.int64))
    tokens = kw.pop("tokens", np.zeros((B, L), np.int64))
    committed = kw.pop("committed", np.zeros((B, L), np.int64))
    done = kw.pop("done", np.zeros(B, np.int64))
    return sampler_step(logits, step, cfg, P, tokens, committed, done, **kw)


def _peak_logits(V, heights, T, ids=None):
    """Logits [1, L, V] with one peak per position; heights chosen in units of
    the target maxprob via the two-level closed form."""
    L = len(heights)
    x = np.zeros((1, L, V))
    ids = ids if ids is not None else np.arange(L) * 7 % V
    for i, a in enumerate(heights):
        x[0, i, ids[i]] = a
    return x, ids


def _height_for_maxprob(p, T, V):
    # maxprob = e^(a/T) / (e^(a/T) + V - 1)  ->  a = T ln(p (V - 1) / (1 - p))
    return T * np.log(p * (V - 1) / (1 - p))


def test_update_rules_planted():
    V, S = 512, 8
    cfg = SamplerCfg(canvas_len=6, max_steps=S, seed=5)
    T = temperature(0, S)
    targets = [0.97, 0.95, 0.5, 0.3, 0.05, 0.02]
    heights = [_height_for_maxprob(p, T, V) for p in targets]
    x, ids = _peak_logits(V, heights, T)
    r = _one_step(x, 0, cfg)
    assert np.allclose(r["maxprob"][0], targets, atol=1e-12)
    assert list(r["committed"][0]) == [1, 1, 0, 0, 0, 0]
    assert list(r["renoised"][0]) == [0, 0, 0, 0, 1, 1]
    for i in range(6):
        if i < 4:
            assert r["tokens"][0, i] == r["sample"][0, i]
        else:
            assert r["tokens"][0, i] == renoise_id(5, i, 0, 0, V)
    assert r["done"][0] == 0

    # committed positions are sticky at the next step, even if unconfident
    x2 = np.zeros_like(x)
    r2 = _one_step(x2, 1, cfg, tokens=r["tokens"], committed=r["committed"])
    assert list(r2["tokens"][0, :2]) == list(r["tokens"][0, :2])
    assert list(r2["committed"][0]) == [1, 1, 0, 0, 0, 0]
    assert list(r2["renoised"][0]) == [0, 0, 1, 1, 1, 1]       # flat -> 1/V


def test_final_step_never_renoises():
    V, S = 512, 8
    cfg = SamplerCfg(canvas_len=4, max_steps=S, seed=1)
    x = np.zeros((1, 4, V))                    # maxprob = 1/V < 0.1
    r = _one_step(x, S - 1, cfg)
    assert r["done"][0] == 1 and r["ends"][0] == 1
    assert r["renoised"].sum() == 0
    assert np.array_equal(r["tokens"], r["sample"])
    r = _one_step(x, S - 2, cfg)
    assert r["done"][0] == 0 and r["renoised"].sum() == 4


def test_adaptive_stop_exact_step():
    """A sequence of logits whose mean entropy crosses the threshold at s*."""
    V, S, L = 512, 48, 8
    cfg = SamplerCfg(canvas_len=L, max_steps=S, seed=3)
    s_star = 5
    tokens = np.zeros((1, L), np.int64)
    committed = np.zeros((1, L), np.int64)
    done = np.zeros(1, np.int64)
    for s in range(S):
        T = temperature(s, S)
        # entropy ~0.041 per position before s*, ~2e-7 from s* on
        a = 12.0 * T if s < s_star else 25.0 * T
        x = np.zeros((1, L, V))
        x[0, :, 0] = a
        r = sampler_step(x, s, cfg, np.zeros(1, np.int64), tokens, committed, done)
        tokens, committed, done = r["tokens"], r["committed"], r["done"]
        if s < s_star:
            assert r["mean_entropy"][0] > cfg.stop_entropy and done[0] == 0
        else:
            assert r["mean_entropy"][0] < cfg.stop_entropy
            assert done[0] == 1 and r["renoised"].sum() == 0
            break
    assert s == s_star


def test_done_rows_untouched():
    V = 512
    cfg = SamplerCfg(canvas_len=3, max_steps=8, seed=2)
    x = np.zeros((2, 3, V))
    tok = np.array([[1, 2, 3], [4, 5, 6]])
    prev = dict(renoised=np.full((2, 3), 7), maxprob=np.full((2, 3), 0.5),
                entropy=np.full((2, 3), 0.25), mean_entropy=np.array([9.0, 9.0]))
    r = sampler_step(x, 0, cfg, np.zeros(2, np.int64), tok, np.zeros((2, 3)),
                     np.array([1, 0]), **prev)
    assert list(r["tokens"][0]) == [1, 2, 3]
    assert list(r["renoised"][0]) == [7, 7, 7]
    assert r["mean_entropy"][0] == 9.0 and r["done"][0] == 1
    assert r["renoised"][1].sum() == 3 and r["done"][1] == 0


def test_fixed_steps_mode():
    V = 512
    cfg = SamplerCfg(canvas_len=4, max_steps=48, fixed_steps=12, seed=4)
    x = np.zeros((1, 4, V))
    x[0, :, 0] = 50.0                          # H ~ 0 < threshold: ignored
    r = _one_step(x, 3, cfg)
    assert r["done"][0] == 0
    assert r["temperature"] == temperature(3, 48)
    x = np.zeros((1, 4, V))
    r = _one_step(x, 11, cfg)
    assert r["done"][0] == 1 and r["renoised"].sum() == 0


def test_gumbel_max_low_temperature_is_argmax():
    V = 64
    cfg = SamplerCfg(canvas_len=5, max_steps=2, temp_start=1e-3, temp_end=1e-3)
    rng = np.random.default_rng(7)
    x = np.stack([rng.permutation(V).astype(np.float64) for _ in range(5)])[None]
    r = _one_step(x, 0, cfg)
    assert np.array_equal(r["sample"][0], x[0].argmax(axis=1))


def test_gumbel_max_frequencies_match_softmax():
    """Empirical distribution of the Gumbel-max sample over many counters
    equals softmax(logits / T) (chi-square, V = 8)."""
    V, L = 8, 4000
    logits = np.array([0.0, 0.5, -1.0, 1.5, 0.2, -0.3, 1.0, 0.0])
    T = 0.8
    cfg = SamplerCfg(canvas_len=L, max_steps=2, temp_start=T, temp_end=T,
                     commit_prob=2.0, renoise_prob=-1.0, seed=11)
    x = np.broadcast_to(logits, (1, L, V)).copy()
    counts = np.zeros(V)
    for rep in range(6):
        r = _one_step(x, 0, cfg, P=np.array([rep * L]))
        counts += np.bincount(r["sample"][0], minlength=V)
    p = np.exp(logits / T)
    p /= p.sum()
    expect = counts.sum() * p
    stat = ((counts - expect) ** 2 / expect).sum()
    assert stat < chi2_dist.ppf(0.9999, V - 1)


def test_init_canvas_uses_stream2():
    tok, com = init_canvas(0, np.array([32, 40]), 4, 512)
    assert com.sum() == 0
    for b, P in enumerate((32, 40)):
        for i in range(4):
            assert tok[b, i] == canvas_id(0, P + i, b, 512)
    assert tok.min() >= 0 and tok.max() < 512


# ---------------------------------------------------- entropy-bound policy (R31)

def test_entropy_bound_select_is_the_largest_feasible_set():
    """Brute force over every subset of the uncommitted positions: the
    selection has the largest size among the sets with sum - max <= bound,
    and it holds the lowest-entropy positions (ties to the lower position)."""
    from itertools import combinations
    from oracle.sampler import entropy_bound_select
    rng = np.random.default_rng(8)
    for trial in range(60):
        L = 7
        h = rng.exponential(0.08, L) if trial % 3 else np.round(rng.exponential(0.08, L), 2)
        com = rng.random(L) < 0.25
        bound = [0.0, 0.05, 0.1, 0.3][trial % 4]
        sel = entropy_bound_select(h, com, bound)
        free = [i for i in range(L) if not com[i]]
        assert not np.any(sel & com)
        best = 0
        for n in range(1, len(free) + 1):
            # sum - max as the sum of all but the largest (no cancellation)
            if any(sum(sorted(h[list(c)])[:-1]) <= bound for c in combinations(free, n)):
                best = n
        assert sel.sum() == best
        if best:
            ranked = sorted(free, key=lambda i: (h[i], i))
            assert set(np.flatnonzero(sel)) == set(ranked[:best])


def _eb_cfg(**kw):
    return SamplerCfg(commit_policy=1, **kw)


def test_entropy_bound_step_planted():
    """Three confident positions (entropy about 1e-3 each, from the two-level
    closed form) and five flat ones: the three plus the lowest flat position
    commit (the largest entropy of the set is not counted against the bound);
    the other flat ones are re-noised (maxprob 1/V < 0.1)."""
    V, S, L = 512, 8, 8
    cfg = _eb_cfg(canvas_len=L, max_steps=S, seed=5)
    T = temperature(0, S)
    x = np.zeros((1, L, V))
    x[0, 2, 7] = x[0, 5, 11] = x[0, 6, 3] = 16.0 * T
    r = _one_step(x, 0, cfg)
    W = np.exp(16.0) + V - 1
    h_conf = np.log(W) - np.exp(16.0) / W * 16.0
    assert np.allclose(r["entropy"][0, [2, 5, 6]], h_conf, rtol=1e-12)
    assert 3 * h_conf < cfg.entropy_bound
    assert list(r["committed"][0]) == [1, 0, 1, 0, 0, 1, 1, 0]
    assert list(r["renoised"][0]) == [0, 1, 0, 1, 1, 0, 0, 1]
    assert r["done"][0] == 0


def test_entropy_bound_commits_all_and_ends():
    V, S, L = 512, 8, 6
    x = np.random.default_rng(1).standard_normal((1, L, V))
    r = _one_step(x, 0, _eb_cfg(canvas_len=L, max_steps=S, seed=2, entropy_bound=1e9))
    assert r["committed"].all() and r["done"][0] == 1 and r["renoised"].sum() == 0
    assert np.array_equal(r["tokens"], r["sample"])
    # fixed steps: no early end
    r = _one_step(x, 0, _eb_cfg(canvas_len=L, max_steps=S, seed=2, entropy_bound=1e9,
                                fixed_steps=4))
    assert r["committed"].all() and r["done"][0] == 0


def test_entropy_bound_zero_commits_one_per_step():
    V, S, L = 512, 8, 5
    cfg = _eb_cfg(canvas_len=L, max_steps=S, seed=3, entropy_bound=0.0, renoise_prob=0.0)
    rng = np.random.default_rng(4)
    tokens = np.zeros((1, L), np.int64)
    committed = np.zeros((1, L), np.int64)
    done = np.zeros(1, np.int64)
    for s in range(L):
        x = rng.standard_normal((1, L, V)) * 3
        r = sampler_step(x, s, cfg, np.zeros(1, np.int64), tokens, committed, done)
        new = r["committed"][0] - committed[0]
        assert new.sum() == 1
        free = np.flatnonzero(committed[0] == 0)
        assert np.flatnonzero(new)[0] == free[np.argmin(r["entropy"][0, free])]
        tokens, committed, done = r["tokens"], r["committed"], r["done"]
        assert done[0] == (1 if s == L - 1 else 0)          # all committed -> ends
