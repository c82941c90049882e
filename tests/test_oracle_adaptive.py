"""Pins for the content-adaptive kept-block count in the oracle.

The pages name sparsity that follows the input as future work and give no rule
(TurboDiffusion explainer, news.qq.com, section on the method's limits, sixth challenge).
The reading checked here: query block i needs the fewest key blocks, taken in selection
order (score descending, lower index on ties), whose pooled mass n_j exp(s_ij - max_j s_ij)
reaches tau of the row's total; a head keeps clamp(ceil(mean_i k_i), kmin, kmax) blocks.
Pins: closed forms for equal and two-level scores (with a ragged last block), a dominant
block, tau = 1, monotonicity in tau, invariance under row shifts and block permutations,
brute force over subsets on tiny rows, and the whole-head forward reducing to the
fixed-count forward at the head's count.
"""
import itertools
import math

import numpy as np
import pytest

import oracle as O


def _bits(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def _lens(N, blk=64):
    Nb = O.num_blocks(N, blk)
    return np.array([min(blk, N - j * blk) for j in range(Nb)], np.float64)


@pytest.mark.parametrize("Nb,tau", [(10, 0.5), (10, 0.55), (37, 0.9), (64, 0.1), (64, 0.25)])
def test_equal_scores_full_blocks(Nb, tau):
    # every block carries the same mass: the count is ceil(tau Nb)
    s = np.full((3, Nb), 0.75)
    k, _ = O.adaptive_k(s, Nb * 64, tau)
    assert (k == math.ceil(tau * Nb - 1e-12)).all()


def test_equal_scores_ragged_last_block_goes_last():
    # equal scores: the lower index comes first, so the short last block (10 tokens) is
    # taken last; W = 9*64 + 10
    N, Nb = 9 * 64 + 10, 10
    s = np.zeros((1, Nb))
    for tau, want in [(0.5, 5), (9 * 64 / (9 * 64 + 10) - 1e-9, 9), (9 * 64 / (9 * 64 + 10) + 1e-6, 10)]:
        k, _ = O.adaptive_k(s, N, tau)
        assert k[0] == want, (tau, k[0], want)


@pytest.mark.parametrize("m,delta,tau", [(3, 2.0, 0.5), (3, 2.0, 0.8), (5, 0.7, 0.95), (1, 4.0, 0.3)])
def test_two_level_closed_form(m, delta, tau):
    # m blocks at score a (mass 64 each), the rest at a - delta (mass 64 e^-delta each),
    # spread over the row
    Nb = 40
    rng = np.random.default_rng(7)
    hi = rng.choice(Nb, m, replace=False)
    row = np.full(Nb, 1.25 - delta)
    row[hi] = 1.25
    W = 64.0 * (m + (Nb - m) * math.exp(-delta))
    T = tau * W
    if T <= 64.0 * m:
        want = math.ceil(T / 64.0 - 1e-12)
    else:
        want = m + math.ceil((T - 64.0 * m) / (64.0 * math.exp(-delta)) - 1e-12)
    k, margin = O.adaptive_k(row[None], Nb * 64, tau)
    assert k[0] == want
    assert margin[0] > 1e-9


def test_dominant_block_needs_one():
    s = np.full((4, 50), -60.0)
    s[np.arange(4), [0, 17, 49, 3]] = 0.0
    for tau in (0.1, 0.5, 0.99):
        k, _ = O.adaptive_k(s, 50 * 64, tau)
        assert (k == 1).all()


def test_tau_one_keeps_every_block_with_mass():
    rng = np.random.default_rng(1)
    s = rng.normal(0, 2, size=(6, 33))
    k, _ = O.adaptive_k(s, 33 * 64 - 5, 1.0)
    assert (k == 33).all()


def test_monotone_in_tau_and_shift_and_permutation_invariant():
    rng = np.random.default_rng(2)
    Nb = 48
    s = rng.integers(-40, 40, size=(8, Nb)).astype(np.float64) / 8.0  # exact in binary
    taus = [0.05, 0.1, 0.3, 0.5, 0.7, 0.9, 0.99]
    ks = [O.adaptive_k(s, Nb * 64, t)[0] for t in taus]
    for a, b in zip(ks, ks[1:]):
        assert (a <= b).all()
    base = ks[3]
    shifted, _ = O.adaptive_k(s + 3.0, Nb * 64, 0.5)  # exact shift of every row
    assert (shifted == base).all()
    # permuting the key blocks (all full, so n_j equal) keeps the count wherever the scores
    # at the decision are distinct
    perm = rng.permutation(Nb)
    sp = s[:, perm]
    kp, _ = O.adaptive_k(sp, Nb * 64, 0.5)
    for i in range(s.shape[0]):
        srt = np.sort(s[i])[::-1]
        kk = base[i]
        if kk < Nb and srt[kk - 1] == srt[kk]:
            continue
        assert kp[i] == base[i]


def test_brute_force_over_subsets():
    # tiny rows: the count is the size of the smallest subset whose mass reaches tau W
    # among subsets that are prefixes of the selection order; brute force over all
    # subsets confirms that no smaller subset of the top blocks would do, and that the
    # chosen prefix is the one with the highest scores
    rng = np.random.default_rng(3)
    N, Nb = 7 * 64 - 20, 7
    n = _lens(N)
    for trial in range(40):
        row = rng.normal(0, 1.5, size=Nb)
        if trial % 5 == 0:
            row[2] = row[5]  # a tie
        tau = rng.uniform(0.05, 0.999)
        w = n * np.exp(row - row.max())
        W = math.fsum(w)
        best = None
        for size in range(1, Nb + 1):
            # the prefix of the selection order of this size: the subsets of this size
            # that beat every other subset of the size on (score, -index) in lexicographic
            # rank order are exactly one, found as the max over all subsets
            cands = list(itertools.combinations(range(Nb), size))
            top = max(cands, key=lambda c: sorted(((row[j], -j) for j in c), reverse=True))
            if math.fsum(w[list(top)]) >= tau * W:
                best = size
                break
        k, margin = O.adaptive_k(row[None], N, tau)
        if margin[0] > 1e-12:
            assert k[0] == best, (trial, k[0], best)


def test_margin_flags_the_decision_distance():
    # two equal blocks and tau exactly one half: the prefix after one block sits on tau W
    s = np.array([[0.0, 0.0]])
    k, margin = O.adaptive_k(s, 128, 0.5)
    assert k[0] == 1 and margin[0] == 0.0
    k, margin = O.adaptive_k(s, 128, 0.25)
    assert k[0] == 1 and abs(margin[0] - 0.25) < 1e-15


def test_head_count_integer_ceiling_and_clamps():
    assert O.adaptive_ksel(np.array([1, 2, 3]), 1, 10) == 2
    assert O.adaptive_ksel(np.array([1, 2, 4]), 1, 10) == 3  # 7/3 -> 3
    assert O.adaptive_ksel(np.array([5] * 7), 1, 10) == 5
    assert O.adaptive_ksel(np.array([30] * 3), 1, 10) == 10
    assert O.adaptive_ksel(np.array([1] * 3), 4, 10) == 4
    # a sum that is a multiple of the count stays exact
    assert O.adaptive_ksel(np.array([3, 3, 3, 3, 3, 3, 3, 3, 3, 3]), 1, 100) == 3


@pytest.mark.parametrize("linear", [False, True])
def test_head_adaptive_reduces_to_fixed_count(linear):
    # the adaptive forward at the head's count equals the fixed-count forward at that count
    rng = np.random.default_rng(4)
    N, d = 11 * 64 - 23, 128
    q = _bits(rng.normal(0, 1, (N, d)))
    k = _bits(rng.normal(0, 1, (N, d)) + rng.normal(0, 2, (1, d)))
    v = _bits(rng.normal(0, 1, (N, d)))
    w = _bits(rng.normal(0, 0.1, (d, d))) if linear else None
    Nb = O.num_blocks(N, 64)
    r = O.sagesla_head_adaptive(q, k, v, w, 0.1, 0.7, 0.6)
    ks = r["ksel"]
    assert O.ksel(0.1, Nb) <= ks <= O.ksel(0.7, Nb)
    # the count follows from the rows' counts of the scores
    qb = O.pool(q, 64)
    kb = O.pool(k, 64)
    S = O.scores(qb, kb)
    kr, _ = O.adaptive_k(S, N, 0.6)
    assert (kr == r["k_rows"]).all()
    assert ks == O.adaptive_ksel(kr, O.ksel(0.1, Nb), O.ksel(0.7, Nb))
    f = O.sagesla_head(q, k, v, w, ks / Nb)
    assert f["ksel"] == ks
    assert np.array_equal(r["out"], f["out"])
    kmax = O.ksel(0.7, Nb)
    assert r["idx"].shape == (Nb, kmax)
    assert np.array_equal(r["idx"][:, :ks], f["idx"])
    assert (r["idx"][:, ks:] == -1).all()
