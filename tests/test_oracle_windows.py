"""Pins of the oracle's WindowQuant steps (W1 scores, W2 bit-width assignment).

WindowQuant notes ("論文メモ：動画VLMのKV Cacheを軽量化するWindowQuant"): the video's
tokens are split into 32-token windows, each window is scored by cosine similarity to
the text query, high / middle / low relevance get FP16 / INT4 / INT2, the first window
stays FP16 whatever its score, and windows of one bit-width are stored together.

Pins: keys built so each window's mean has a chosen angle to the text vector (so the
cosine is known in closed form), the assignment compared with numpy's lexsort, the
budget of the 100-frame workload (61 / 184 / 368), the short tail window, and ties.
"""
import numpy as np
import pytest

import workloads


def _construct(rng, W, H, d, window, N, text):
    """Keys whose window means are r_w (cos th_w t^ + sin th_w u_w): cosine = cos th_w."""
    th = rng.permutation(np.linspace(0.05, 3.0, W))
    that = text / np.linalg.norm(text)
    K = np.zeros((H, N, d), np.float64)
    for h in range(H):
        for w in range(W):
            u = rng.standard_normal(d)
            u -= (u @ that) * that
            u /= np.linalg.norm(u)
            mean = rng.uniform(0.5, 2.0) * (np.cos(th[w]) * that + np.sin(th[w]) * u)
            t0, t1 = w * window, min(N, w * window + window)
            n = t1 - t0
            dev = rng.standard_normal((n, d)) * 0.25
            dev -= dev.mean(0)
            K[h, t0:t1] = mean + dev
    return K.astype(np.float32), np.cos(th)


def test_known_cosines(orc):
    rng = np.random.default_rng(1)
    d, H, window = 64, 2, 32
    N = 40 * 32 - 16                        # tail window of 16 tokens
    W = -(-N // window)
    text = rng.standard_normal(d).astype(np.float32)
    K, cos = _construct(rng, W, H, d, window, N, text)
    s = orc.window_scores(K, text, window)
    assert s.shape == (W,)
    np.testing.assert_allclose(s, cos, atol=2e-6)       # float32 keys: ~1e-7 of rounding
    # exact definition of the score on one window, computed independently in numpy
    w = W - 1
    m = K[:, w * window:].astype(np.float64).mean(1)    # [H][d]; tail window: 16 tokens
    t = text.astype(np.float64)
    want = np.mean([m[h] @ t / (np.linalg.norm(m[h]) * np.linalg.norm(t)) for h in range(H)])
    np.testing.assert_allclose(s[w], want, rtol=1e-13)


def test_assignment_matches_lexsort(orc):
    rng = np.random.default_rng(2)
    for W in (1, 2, 7, 100, 613):
        score = rng.standard_normal(W)
        score[0] = score.min() - 1                       # window 0 least relevant
        n16, n4 = orc.window_budget(W, 10, 30)
        bits, order = orc.assign_windows(score, n16, n4)
        assert bits[0] == 16
        rest = np.arange(1, W)
        ranked = rest[np.lexsort((rest, -score[1:]))]
        want = np.full(W, 2, np.int8)
        want[0] = 16
        want[ranked[:n16 - 1]] = 16
        want[ranked[n16 - 1:n16 - 1 + n4]] = 4
        assert np.array_equal(bits, want)
        want_order = np.concatenate([np.nonzero(want == b)[0] for b in (16, 4, 2)])
        assert np.array_equal(order, want_order)
        assert (bits == 16).sum() == n16 and (bits == 4).sum() == n4


def test_windowquant_workload_budget(orc):
    w = workloads.WORKLOADS["windowquant_fp16_gqa14x2_d64"]
    assert w.n_windows == 613
    n16, n4 = orc.window_budget(w.n_windows, w.pct_fp16, w.pct_int4)
    assert (n16, n4, w.n_windows - n16 - n4) == (61, 184, 368)
    assert orc.window_budget(5, 10, 30) == (1, 2)        # floor 0 FP16 raised to window 0


def test_ties_go_to_lower_index(orc):
    score = np.array([0.0, 0.5, 0.9, 0.5, 0.9, 0.1])
    bits, order = orc.assign_windows(score, 2, 2)     # one FP16 slot besides window 0
    assert list(bits) == [16, 4, 16, 2, 4, 2]
    assert list(order) == [0, 2, 1, 4, 3, 5]


def test_zero_vectors_score_zero(orc):
    K = np.zeros((2, 64, 64), np.float32)
    K[:, 32:] = 1.0
    text = np.ones(64, np.float32)
    s = orc.window_scores(K, text, 32)
    assert s[0] == 0.0 and s[1] == pytest.approx(1.0, abs=1e-15)
    assert np.all(orc.window_scores(K, np.zeros(64, np.float32), 32) == 0.0)


def test_grouped_layout_lists(orc):
    """A6: the gather lists cover every token exactly once, FP16 windows first, then INT4,
    then INT2, ascending inside each class; the short last window counts its own length;
    the class token counts add up to N. Hand case: 5 windows of 4 tokens over N = 18."""
    bits = np.array([16, 2, 4, 16, 2], np.int8)
    order = np.array([0, 3, 2, 1, 4], np.int32)
    groups, ct = orc.window_groups(bits, order, 18, 4)
    assert groups.tolist() == [[0, 4], [12, 4], [8, 4], [4, 4], [16, 2]]
    assert ct.tolist() == [8, 4, 6]
    rng = np.random.default_rng(7)
    for N in (19600, 19599, 32, 33):
        W = -(-N // 32)
        score = rng.standard_normal(W)
        n16, n4 = orc.window_budget(W, 10, 30)
        b, o = orc.assign_windows(score, n16, n4)
        g, ct = orc.window_groups(b, o, N, 32)
        covered = np.zeros(N, np.int32)
        for s0, ln in g:
            covered[s0:s0 + ln] += 1
        assert np.all(covered == 1)
        assert ct.sum() == N
        bounds = np.cumsum([0, n16, n4, W - n16 - n4])
        for k, cls in enumerate((16, 4, 2)):
            rows = g[bounds[k]:bounds[k + 1]]
            assert np.all(np.diff(rows[:, 0]) > 0)
            assert np.all(b[rows[:, 0] // 32] == cls)
            assert rows[:, 1].sum() == ct[k]
