"""The accuracy measurement's definitions (host float64), pinned by hand-
computable cases: exact top-k against a brute-force sort with ties, softmax
attention with a zero query (uniform weights), and the error and recall of
identical and disjoint selections."""
import numpy as np

from sparse_attention_key_amd import accuracy as A


def test_exact_topk_brute_force_with_ties():
    g = np.random.default_rng(3)
    s = np.round(g.standard_normal((3, 200)) * 2) / 2  # many ties
    got = A.exact_topk(s, 17)
    for h in range(3):
        order = sorted(range(200), key=lambda i: (-s[h, i], i))[:17]
        assert list(got[h]) == order


def test_attention_with_zero_query_is_the_mean():
    g = np.random.default_rng(4)
    keys = g.standard_normal((10, 4))
    vals = g.standard_normal((10, 4))
    o = A.attention(np.zeros(4), keys, vals, [1, 3, 8])
    assert np.allclose(o, vals[[1, 3, 8]].mean(0), rtol=0, atol=1e-15)


def test_attention_two_tokens_by_hand():
    keys = np.array([[2.0, 0.0], [0.0, 0.0]])
    vals = np.array([[1.0, 0.0], [0.0, 1.0]])
    q = np.array([np.sqrt(2.0) * np.log(3.0) / 2.0, 5.0])  # score gap log(3) after /sqrt(2)
    o = A.attention(q, keys, vals, [0, 1])
    assert np.allclose(o, [0.75, 0.25], atol=1e-14)


def test_metrics_identical_and_disjoint():
    keys = np.zeros((4, 2))
    vals = np.array([[1.0, 0.0], [1.0, 0.0], [0.0, 1.0], [0.0, 3.0]])
    q = np.zeros((1, 2))
    e, r = A.selection_metrics(q, keys, vals, np.array([[0, 1]]), np.array([[1, 0]]))
    assert e[0] == 0.0 and r[0] == 1.0
    # uniform weights: o_S = (1, 0), o_ref = (0, 2): error ||(1, -2)|| / 2
    e, r = A.selection_metrics(q, keys, vals, np.array([[0, 1]]), np.array([[2, 3]]))
    assert np.isclose(e[0], np.sqrt(5.0) / 2.0) and r[0] == 0.0


def test_plan_spec_parsing():
    assert A.parse_plan("B48") == ("waterfill", 48)
    assert A.parse_plan("r16") == ("topr", 16)
    assert A.parse_plan("u2") == ("uniform", 2)
