"""Pins for pooling, scoring and top-k block selection in the oracle.

SLA first scores how strongly pairs are related and keeps only the top fraction
(TurboDiffusion explainer, news.qq.com, section "First key: attention"). The kept set
per query block is checked against an exhaustive sort (numpy lexsort) and, on tiny
inputs, against brute force over all subsets; the count against the pages' Top-K ratios.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bits(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_ksel_matches_pages_ratios():
    g = json.load(open(os.path.join(GOLD, "topk_pages.json")))
    for c in g["cases"]:
        Nb = O.num_blocks(c["N"], 64)
        assert Nb == c["Nb"]
        assert O.ksel(c["topk"], Nb) == c["ksel"], c


def test_ksel_bounds():
    for Nb in (1, 2, 7, 30, 512, 1182):
        assert O.ksel(1e-9, Nb) == 1
        assert O.ksel(1.0, Nb) == Nb
        for t in (0.05, 0.1, 0.15, 0.25, 0.5):
            k = O.ksel(t, Nb)
            assert 1 <= k <= Nb
            assert k >= t * Nb - 1e-6  # at least the requested fraction
            assert k == 1 or k - 1 < t * Nb - 1e-12  # and the smallest such count


def test_pool_block_means_with_partial_block():
    # block i holds the constant i+1 in every channel; last block has 5 valid tokens
    N, d = 64 * 3 + 5, 16
    x = np.zeros((N, d), np.float32)
    for t in range(N):
        x[t] = t // 64 + 1
    x[-5:, 3] = np.arange(5)  # mean 2.0 over the 5 valid tokens
    m = O.pool(_bits(x), 64)
    assert m.shape == (4, d)
    assert np.all(m[:3] == np.arange(1, 4)[:, None])
    assert m[3, 0] == 4.0 and m[3, 3] == 2.0


def _exhaustive(s, k):
    out = []
    for row in s:
        order = np.lexsort((np.arange(len(row)), -row))  # score desc, then index asc
        out.append(np.sort(order[:k]))
    return np.array(out, np.int32)


@pytest.mark.parametrize("Nb,k,seed,grid", [(32, 4, 0, None), (31, 7, 1, None), (20, 20, 2, None),
                                              (16, 5, 3, 0.5), (25, 1, 4, 0.25)])
def test_select_equals_exhaustive_sort(Nb, k, seed, grid):
    rng = np.random.default_rng(seed)
    s = rng.normal(size=(Nb, Nb))
    if grid:  # coarse grid -> many exact ties, exercising the lower-index rule
        s = np.round(s / grid) * grid
    got = O.select(s, k)
    assert np.array_equal(got, _exhaustive(s, k))
    assert np.all(np.diff(got, axis=1) > 0)  # ascending


def test_select_equals_brute_force_subsets():
    rng = np.random.default_rng(11)
    for Nb in (3, 5, 8):
        for k in range(1, Nb + 1):
            s = rng.normal(size=(Nb, Nb))
            got = O.select(s, k)
            for i in range(Nb):
                best = max(itertools.combinations(range(Nb), k), key=lambda c: s[i, list(c)].sum())
                assert tuple(got[i]) == best


def test_scores_closed_form_unit_vectors():
    d = 128
    qbar = np.zeros((3, d))
    kbar = np.zeros((3, d))
    qbar[0, 5] = 2.0
    qbar[1, 7] = -1.0
    qbar[2, :] = 1.0
    kbar[0, 5] = 3.0
    kbar[1, 7] = 4.0
    kbar[2, 9] = 1.0
    s = O.scores(qbar, kbar)
    r = math.sqrt(d)
    want = np.array([[6, 0, 0], [0, -4, 0], [3, 4, 1]]) / r
    assert np.allclose(s, want, rtol=0, atol=1e-15)


def _mask_of(q, k, topk):
    qb, kb = O.pool(q), O.pool(k)
    s = O.scores(qb, kb)
    return O.select(s, O.ksel(topk, qb.shape[0])), s


def test_mask_invariances():
    """A per-channel constant added to K, or a positive scale on Q, leaves the kept set."""
    rng = np.random.default_rng(5)
    N, d = 64 * 12 + 17, 128
    q = rng.normal(size=(N, d)).astype(np.float32)
    k = rng.normal(size=(N, d)).astype(np.float32)
    # values on a 1/16 grid in [-4, 4] so that +8 and *2 are exact in bf16
    q = np.clip(np.round(q * 16) / 16, -4, 4)
    k = np.clip(np.round(k * 16) / 16, -4, 4)
    base, s = _mask_of(_bits(q), _bits(k), 0.25)
    off = np.zeros(d, np.float32)
    off[::3] = 8.0
    shifted, _ = _mask_of(_bits(q), _bits(k + off), 0.25)
    scaled, _ = _mask_of(_bits(q * 2), _bits(k), 0.25)
    assert np.array_equal(base, scaled)
    # the shift adds qbar_i . off / sqrt(d) to a whole row: same set unless a near-tie
    diff = [i for i in range(len(base)) if not np.array_equal(base[i], shifted[i])]
    for i in diff:
        row = np.sort(s[i])[::-1]
        kk = base.shape[1]
        assert abs(row[kk - 1] - row[kk]) < 1e-9


def test_processing_order_best_first_then_ascending():
    rng = np.random.default_rng(12)
    for trial in range(50):
        Nb = int(rng.integers(2, 40))
        row = rng.normal(size=Nb)
        if trial % 3 == 0:
            row = np.round(row * 2) / 2  # ties
        k = int(rng.integers(1, Nb + 1))
        kept = O.select(row[None, :], k)[0]
        got = O.order_best_first(row, kept)
        best = kept[np.lexsort((kept, -row[kept]))[0]]  # highest score, lowest index
        assert got[0] == best
        assert list(got[1:]) == sorted(set(kept.tolist()) - {best})
