"""Pins of the oracle's sampler (sample_next) to closed forms.

- temperature 0 and top_k 1 take the argmax (ties to the lower id);
- k equal logits at temperature 1: the draw u picks candidate floor(u k),
  and the candidates are the k lowest ids;
- two candidates a logit gap d apart: the better one exactly while
  u < 1 / (1 + exp(-d / T));
- top-p and min-p on the probabilities 0.5, 0.3, 0.2: the kept sets written
  out by hand, and the renormalised split point of u;
- top_k outside 1 .. 64 keeps 64 candidates;
- on a grid of N draws every token's frequency is its kept probability,
  renormalised, at temperature T (p^(1/T) renormalised), within 1/N.
"""
import math

import pytest
import torch

import oracle as O


def logits_of(probs, pad=0):
    z = torch.log(torch.tensor(probs, dtype=torch.float64))
    return torch.cat([z, torch.full((pad,), -1e30, dtype=torch.float64)])


def test_greedy_cases():
    z = torch.tensor([0.5, 2.0, 2.0, -1.0])
    assert O.sample_next(z, 0.0, 40, 0.9, 0.0, 0.7) == 1
    assert O.sample_next(z, -1.0, 40, 1.0, 0.0, 0.7) == 1
    assert O.sample_next(z, 1.5, 1, 1.0, 0.0, 0.99) == 1


@pytest.mark.parametrize("k", [2, 5, 64])
def test_equal_logits_split_u_evenly(k):
    z = torch.zeros(200)
    for i in range(k):
        u = (i + 0.5) / k
        assert O.sample_next(z, 1.0, k, 1.0, 0.0, u) == i


@pytest.mark.parametrize("d,T", [(1.0, 1.0), (2.0, 0.5), (0.3, 2.0)])
def test_two_candidates(d, T):
    z = torch.tensor([0.0, d, -50.0], dtype=torch.float64)
    p_best = 1.0 / (1.0 + math.exp(-d / T))
    assert O.sample_next(z, T, 2, 1.0, 0.0, p_best - 1e-9) == 1
    assert O.sample_next(z, T, 2, 1.0, 0.0, p_best + 1e-9) == 0


def test_top_p_and_min_p_by_hand():
    z = logits_of([0.5, 0.3, 0.2])
    # top_p 0.6: 0.5 < 0.6 <= 0.8, so tokens 0 and 1, split at 0.5 / 0.8
    assert O.sample_next(z, 1.0, 3, 0.6, 0.0, 0.62) == 0
    assert O.sample_next(z, 1.0, 3, 0.6, 0.0, 0.63) == 1
    assert O.sample_next(z, 1.0, 3, 0.6, 0.0, 0.999) == 1
    # top_p 0.5 is reached by token 0 alone
    assert O.sample_next(z, 1.0, 3, 0.5, 0.0, 0.999) == 0
    # min_p 0.5: p >= 0.25 keeps tokens 0 and 1; min_p 0.7: only token 0
    assert O.sample_next(z, 1.0, 3, 1.0, 0.5, 0.99) == 1
    assert O.sample_next(z, 1.0, 3, 1.0, 0.7, 0.99) == 0
    # no filter: u past 0.8 lands on token 2
    assert O.sample_next(z, 1.0, 3, 1.0, 0.0, 0.81) == 2


def test_top_k_outside_the_range_keeps_64():
    z = -torch.arange(300, dtype=torch.float64) * 1e-6      # nearly equal, decreasing
    for k in (0, -3, 65, 1000):
        assert O.sample_next(z, 1.0, k, 1.0, 0.0, 0.9999) == 63
    assert O.sample_next(z, 1.0, 10, 1.0, 0.0, 0.9999) == 9


@pytest.mark.parametrize("T,top_p,min_p", [(1.0, 1.0, 0.0), (0.5, 1.0, 0.0), (1.3, 0.9, 0.0),
                                           (0.8, 1.0, 0.1)])
def test_grid_frequencies(T, top_p, min_p):
    probs = [0.3, 0.25, 0.15, 0.12, 0.08, 0.06, 0.04]
    z = logits_of(probs, pad=20)
    # the kept set by hand: top-p prefix, then min-p
    cum, kept = 0.0, []
    for i, p in enumerate(probs):
        kept.append(i)
        cum += p
        if cum >= top_p:
            break
    kept = [i for i in kept if probs[i] >= min_p * probs[0] or i == 0]
    w = [probs[i] ** (1.0 / T) for i in kept]
    want = {i: wi / sum(w) for i, wi in zip(kept, w)}
    N = 4000
    counts = {}
    for j in range(N):
        t = O.sample_next(z, T, 10, top_p, min_p, (j + 0.5) / N)
        counts[t] = counts.get(t, 0) + 1
    assert set(counts) <= set(kept)
    for i in kept:
        assert abs(counts.get(i, 0) / N - want[i]) <= 1.0 / N + 1e-12
