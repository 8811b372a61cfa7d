"""Pins of the region-selection oracle (CPU): a hand-worked golden file, an
exhaustive subset search on tiny rows, numpy's argsort on distinct scores,
closed forms and invariants."""
import itertools
import math
import os

import numpy as np
import pytest

from oracle import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    cases = []
    for line in open(os.path.join(HERE, "golden", "select_regions_example.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        s, cur, k, n, exp = [x.strip() for x in line.split("|")]
        cases.append((np.array([float(x) for x in s.split()], np.float32), int(cur), int(k),
                      int(n), [int(x) for x in exp.split()]))
    return cases


@pytest.mark.parametrize("case", _golden(), ids=lambda c: "k%d-cur%d-n%d" % (c[2], c[1], c[3]))
def test_golden_examples(case):
    s, cur, k, n, exp = case
    lens = None if n < 0 else np.array([n], np.int32)
    got = oracle.select_regions(s[None, :], np.array([cur], np.int32), k, lens)
    assert got[0].tolist() == exp


def _rank_key(x):
    # score order with -0.0 below +0.0
    return (float(x), 0 if math.copysign(1.0, float(x)) < 0 else 1)


def _exhaustive(s, cur, k, n):
    """Among all subsets of the right size, the one whose sorted score keys
    are largest; among equal ones, the smallest sorted id tuple."""
    forced = 0 <= cur < n and k > 0
    cand = [j for j in range(n) if not (forced and j == cur)]
    take = min(max(k - forced, 0), len(cand))
    best = None
    for sub in itertools.combinations(cand, take):
        keys = sorted((_rank_key(s[j]) for j in sub), reverse=True)
        key = (keys, [-j for j in sorted(sub)])
        if best is None or key > best[0]:
            best = (key, sub)
    sel = sorted(list(best[1]) + ([cur] if forced else []))
    return sel + [-1] * (k - len(sel))


@pytest.mark.parametrize("seed", range(300))
def test_exhaustive_search_on_tiny_rows(seed):
    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, 10))
    # few distinct values so that ties are common; signed zeros included
    vals = np.array([-2.0, -0.0, 0.0, 1.0, 1.5, 3.0], np.float32)
    s = rng.choice(vals, size=S).astype(np.float32) if seed % 2 else \
        rng.standard_normal(S).astype(np.float32)
    k = int(rng.integers(0, S + 3))
    n = int(rng.integers(-1, S + 2))
    cur = int(rng.integers(-2, S + 1))
    lens = np.array([n], np.int32)
    got = oracle.select_regions(s[None, :], np.array([cur], np.int32), k, lens)[0].tolist()
    assert got == _exhaustive(s, cur, k, min(max(n, 0), S))


def test_matches_argsort_on_distinct_scores():
    rng = np.random.default_rng(5)
    rows, S, k = 40, 3000, 257
    s = rng.standard_normal((rows, S)).astype(np.float32)
    lens = rng.integers(0, S + 1, size=rows).astype(np.int32)
    cur = np.array([max(int(n) - 1, 0) for n in lens], np.int32)
    got = oracle.select_regions(s, cur, k, lens)
    for r in range(rows):
        n = int(lens[r])
        forced = 0 <= cur[r] < n
        cand = np.array([j for j in range(n) if not (forced and j == cur[r])], np.int64)
        order = cand[np.argsort(-s[r, cand], kind="stable")] if len(cand) else cand
        sel = sorted(order[:k - int(forced)].tolist() + ([int(cur[r])] if forced else []))
        assert got[r].tolist() == sel + [-1] * (k - len(sel))


def test_closed_forms():
    S, k = 100, 10
    idx = np.arange(S, dtype=np.float32)
    # decreasing scores: the lowest ids win; the forced current joins them
    got = oracle.select_regions((-idx)[None, :], np.array([50], np.int32), k)[0]
    assert got.tolist() == list(range(9)) + [50]
    # increasing scores: the highest ids below the length win
    got = oracle.select_regions(idx[None, :], np.array([3], np.int32), k,
                                np.array([60], np.int32))[0]
    assert got.tolist() == [3] + list(range(51, 60))
    # topk >= candidates: every candidate, then -1
    got = oracle.select_regions(idx[None, :], np.array([0], np.int32), 20,
                                np.array([12], np.int32))[0]
    assert got.tolist() == list(range(12)) + [-1] * 8


def test_invariants():
    rng = np.random.default_rng(9)
    rows, S, k = 16, 200, 17
    s = rng.standard_normal((rows, S)).astype(np.float32)
    lens = rng.integers(1, S + 1, size=rows).astype(np.int32)
    cur = (lens - 1).astype(np.int32)
    base = oracle.select_regions(s, cur, k, lens)
    # scores past a row's length do not matter
    s2 = s.copy()
    for r in range(rows):
        s2[r, lens[r]:] = np.inf
    assert np.array_equal(oracle.select_regions(s2, cur, k, lens), base)
    # the forced region is in even with the lowest score
    s3 = s.copy()
    s3[np.arange(rows), cur] = -np.inf
    got = oracle.select_regions(s3, cur, k, lens)
    assert all(int(cur[r]) in got[r] for r in range(rows))
    # raising a selected score keeps the set; an unselected score below the
    # threshold can be lowered further without change
    assert np.array_equal(oracle.select_regions(s + 0.0, cur, k, lens), base)
    # topk = 0: nothing
    assert oracle.select_regions(s, cur, 0, lens).shape == (rows, 0)
    # no lengths: all S columns are candidates
    full = oracle.select_regions(s, cur, k)
    same = oracle.select_regions(s, cur, k, np.full(rows, S, np.int32))
    assert np.array_equal(full, same)
