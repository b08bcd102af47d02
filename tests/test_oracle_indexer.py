"""Pins of the oracle's indexer score and top-k (CPU only).

* Score s_j = sum_h w_h relu(q_h . k_j) (the Ref workload's definition),
  checked by plain Python loops on tiny inputs and by a closed form.
* Selection: the k best causal entries ([vLLM-V4] section 2, DSA top-k;
  appendix, causality 4j + 3 <= t), checked by brute force with Python's
  sorted(), planted winners, and a planted future entry that must never win.
"""

import numpy as np

from oracle import formats, geometry, indexer
from oracle.paged import PagedCache


def loop_scores(q, w, keys):
    out = []
    for k in keys:
        s = 0.0
        for h in range(len(q)):
            dot = sum(float(q[h][i]) * float(k[i]) for i in range(len(k)))
            s += float(w[h]) * max(0.0, dot)
        out.append(s)
    return np.array(out)


def test_scores_match_loops():
    rng = np.random.default_rng(0)
    q, w, keys = rng.standard_normal((4, 16)), rng.uniform(0, 1, 4), rng.standard_normal((30, 16))
    assert np.allclose(indexer.scores(q, w, keys), loop_scores(q, w, keys), rtol=1e-12, atol=1e-12)


def test_scores_closed_form():
    rng = np.random.default_rng(1)
    q1 = rng.standard_normal(8)
    keys = rng.standard_normal((20, 8))
    q = np.tile(q1, (3, 1))
    w = np.array([0.2, 0.3, 0.5])        # identical heads with weights summing to 1: relu(q . k)
    assert np.allclose(indexer.scores(q, w, keys), np.maximum(keys @ q1, 0), atol=1e-12)
    assert np.all(indexer.scores(-q, w, -keys) == indexer.scores(q, w, keys))


def test_topk_brute_force_and_ties():
    rng = np.random.default_rng(2)
    for n, k in [(50, 7), (50, 50), (10, 64), (1, 1), (0, 4)]:
        s = np.round(rng.standard_normal(n), 1)           # many exact ties
        ref = sorted(range(n), key=lambda j: (-s[j], j))[:k]
        got = indexer.topk(s, k)
        assert list(got[:len(ref)]) == ref
        assert np.all(got[len(ref):] == -1)


def test_topk_from_cache_is_causal_and_finds_planted():
    rng = np.random.default_rng(3)
    d, H, L = 128, 4, 1024
    n_all = geometry.num_entries(L, 4)
    cache = PagedCache.empty(1, n_all, 64, d, "fp8", perm_seed=7)
    for j in range(n_all):
        cache.write(0, j, rng.standard_normal(d))
    q, w = rng.standard_normal((H, d)), rng.uniform(0, 1, H)
    t = 803                                               # sees entries j with 4j + 3 <= 803: j < 201
    n = geometry.visible_entries(t, 4)
    assert n == 201
    big = q.sum(axis=0) * 100
    cache.write(0, n, big)                                # first future entry: huge score, must not win
    for j in (5, 77, 200):
        cache.write(0, j, big * (1 + j / 1000))           # planted winners
    sel = indexer.topk(indexer.query_scores(cache, 0, t, q, w), 3)
    assert sorted(sel) == [5, 77, 200]
    keys = formats.fp8_e4m3_to_f64(cache.rows[cache.locate(0, np.arange(n))]) * \
        cache.scales[cache.locate(0, np.arange(n))][:, None]
    assert np.allclose(indexer.query_scores(cache, 0, t, q, w), loop_scores(q, w, keys), rtol=1e-12)
