"""Pins of the reference sampler (oracle/sampling.py) against closed forms, an
independent torch route and the defining properties of each step."""
import numpy as np
import pytest
import torch

from oracle import sampling as S


def test_greedy_is_first_argmax():
    lg = np.array([0.5, 2.0, -1.0, 2.0], dtype=np.float32)
    assert S.sample(lg, 0.0, 40) == 1
    assert S.sample(lg, -1.0, 40, top_p=0.1, repeat_penalty=3.0, recent=[1], u=0.99) == 1  # nothing else applies


def test_top_k_one_is_argmax_of_transformed():
    lg = np.array([2.0, 1.9, -1.0], dtype=np.float32)
    assert S.sample(lg, 1.0, 1, u=0.7) == 0
    # the penalty halves token 0's positive logit: token 1 ranks first
    assert S.sample(lg, 1.0, 1, repeat_penalty=2.0, recent=[0, 0, -1], u=0.7) == 1


def test_penalty_sign_rule():
    z = S.transformed(np.array([3.0, -1.5, 0.5], dtype=np.float32), 1.0, 1.5, recent=[0, 1, 1, 7, -1])
    np.testing.assert_array_equal(z, np.array([2.0, -2.25, 0.5], dtype=np.float32))


def test_temperature_divides_first():
    z = S.transformed(np.array([3.0, -3.0], dtype=np.float32), 2.0, 3.0, recent=[0, 1])
    np.testing.assert_array_equal(z, np.array([0.5, -4.5], dtype=np.float32))


def test_closed_form_three_tokens():
    # probabilities 0.5, 0.3, 0.2: cumulative 0.5, 0.8, 1.0
    lg = np.log(np.array([0.5, 0.3, 0.2])).astype(np.float32)
    for u, want in [(0.0, 0), (0.49, 0), (0.51, 1), (0.79, 1), (0.81, 2), (0.999, 2)]:
        assert S.sample(lg, 1.0, 3, u=u) == want
    # top-p 0.6: the prefix must exceed 0.6, so it is {0, 1}, renormalised to 5/8, 3/8
    for u, want in [(0.6, 0), (0.63, 1)]:
        assert S.sample(lg, 1.0, 3, top_p=0.6, u=u) == want
    tok, ids, cum, tot = S.sample(lg, 1.0, 3, top_p=0.6, u=0.3, detail=True)
    np.testing.assert_array_equal(ids, [0, 1])
    np.testing.assert_allclose(cum / tot, [0.625, 1.0], rtol=1e-6)
    # two equal tokens (exactly 1/2 each): a top-p of exactly 0.5 is not exceeded
    # by the first token, so the second is kept too
    assert len(S.sample(np.zeros(2, np.float32), 1.0, 2, top_p=0.5, detail=True)[1]) == 2
    # a tiny top-p keeps only the first token
    assert S.sample(lg, 1.0, 3, top_p=1e-9, u=0.99) == 0


def test_temperature_closed_form():
    lg = np.array([2.0, 0.0], dtype=np.float32)
    p0 = 1.0 / (1.0 + np.exp(-1.0))  # temperature 2: z = (1, 0)
    assert S.sample(lg, 2.0, 2, u=p0 - 1e-6) == 0
    assert S.sample(lg, 2.0, 2, u=p0 + 1e-6) == 1


def test_ties_take_lower_index():
    lg = np.array([1.0, 0.0, 1.0, 1.0], dtype=np.float32)
    _, ids, _, _ = S.sample(lg, 1.0, 2, detail=True)
    np.testing.assert_array_equal(ids, [0, 2])
    z = S.transformed(np.array([0.0, -0.0, 0.0], dtype=np.float32), 1.0)
    np.testing.assert_array_equal(S.canonical_order(z), [0, 1, 2])  # -0 ranks as +0


def test_against_torch_topk_softmax():
    rng = np.random.default_rng(3)
    lg = (rng.standard_normal(5000) * 2).astype(np.float32)
    for k, p, t in [(1, 1.0, 0.7), (40, 1.0, 1.0), (300, 0.9, 0.8), (4096, 0.95, 1.3)]:
        _, ids, cum, tot = S.sample(lg, t, k, top_p=p, detail=True)
        zt = torch.from_numpy(lg) / torch.tensor(t, dtype=torch.float32)
        vals, tidx = torch.topk(zt.double(), k)
        probs = torch.softmax(vals, 0).numpy()
        c = np.cumsum(probs)
        n_p = int(np.argmax(c > p)) + 1 if p < 1.0 else k
        np.testing.assert_array_equal(ids, tidx.numpy()[:n_p])  # no exact ties in this draw
        np.testing.assert_allclose(cum / cum[-1], c[:n_p] / c[n_p - 1], rtol=1e-9)


def test_draw_frequencies_follow_probabilities():
    rng = np.random.default_rng(4)
    lg = rng.standard_normal(12).astype(np.float32)
    n = 20000
    counts = np.zeros(12)
    for i in range(n):
        counts[S.sample(lg, 1.0, 12, u=(i + 0.5) / n)] += 1
    p = np.exp(lg.astype(np.float64) - lg.max())
    p /= p.sum()
    np.testing.assert_allclose(counts / n, p, atol=2.0 / n)
