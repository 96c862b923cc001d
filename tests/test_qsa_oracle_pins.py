"""Pins of the QSA indexer oracle (oracle/qsa.py) against facts that do not come from the
oracle itself: hand-computed means, the complex-number form of a rotation, the relative-position
property of rotary encodings, softmax invariants and closed forms, causality, and an independent
rank-based definition of top-k.  Each one is chosen so that a plausible slip in the oracle (RoPE
before pooling, a wrong pairing or sign, a softmax over the wrong axis, an off-by-one in the
causal boundary, a wrong tie rule) fails it.
"""
import math

import numpy as np
import pytest

from oracle import qsa


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ---- pooling: keys are averaged per block of r tokens; the last block may be short
def test_pool_hand_example():
    k = np.array([1.0, 2.0, 3.0, 4.0, 10.0]).reshape(1, 5, 1)
    out = qsa.pool_keys(k, 2)
    assert out.shape == (1, 3, 1)
    assert out[0, :, 0].tolist() == [1.5, 3.5, 10.0]
    assert np.array_equal(qsa.pool_keys(k, 1), k)
    assert qsa.pool_keys(k, 8)[0, 0, 0] == 4.0  # one short block: mean of all five


# ---- rotary encoding
def test_rope_equals_complex_multiplication():
    """x[i] + i*x[i+h] turns by exp(i * pos * base^(-2i/R)) for i < h = R/2; the rest is kept."""
    x = rng(1).standard_normal((5, 12))
    pos = np.arange(5) * 7.0
    R, h, base = 8, 4, 500.0
    got = qsa.rope(x, pos, R, base)
    for p in range(5):
        z = x[p, :h] + 1j * x[p, h:R]
        z = z * np.exp(1j * pos[p] * base ** (-2.0 * np.arange(h) / R))
        assert np.allclose(got[p, :h], z.real, atol=1e-13)
        assert np.allclose(got[p, h:R], z.imag, atol=1e-13)
        assert np.array_equal(got[p, R:], x[p, R:])


def test_rope_norm_identity_and_relative_position():
    g = rng(2)
    q, k = g.standard_normal(16), g.standard_normal(16)
    assert np.allclose(np.linalg.norm(qsa.rope(q, 123.0, 16)), np.linalg.norm(q), atol=1e-12)
    assert np.array_equal(qsa.rope(q, 0.0, 16), q)
    assert np.array_equal(qsa.rope(q, 55.0, 0), q)
    # the product of two rotated vectors depends only on the distance of their positions
    a = qsa.rope(q, 40.0, 16) @ qsa.rope(k, 13.0, 16)
    b = qsa.rope(q, 27.0, 16) @ k
    assert math.isclose(a, b, rel_tol=1e-12, abs_tol=1e-12)


# ---- importance
def small_case(seed, B=2, T=37, Hq=4, d=16, scale_q=1.0):
    g = rng(seed)
    return g.standard_normal((B, T, Hq, d)) * scale_q, g.standard_normal((B, T, d))


def test_importance_is_a_sum_of_head_distributions():
    q, k = small_case(3)
    imp, elig = qsa.importance(q, k, r=4, rope_dims=8)
    n = elig.sum(axis=1)
    assert n.tolist() == [(t + 1) // 4 for t in range(36)] + [10]  # 37 tokens: short last block
    tot = imp.sum(axis=2)
    assert np.allclose(tot[:, n > 0], 4.0, atol=1e-12)
    assert np.all(imp[:, n == 0] == 0) and np.all(imp[:, ~elig] == 0)
    assert np.all(imp[:, elig] > 0)


def test_importance_heads_are_independent():
    """Four heads = the sum of four single-head indexers (no softmax across heads)."""
    q, k = small_case(4)
    imp, _ = qsa.importance(q, k, r=3, rope_dims=16)
    parts = sum(qsa.importance(q[:, :, h:h + 1], k, r=3, rope_dims=16)[0] for h in range(4))
    assert np.allclose(imp, parts, atol=1e-13)


def test_importance_two_blocks_closed_form():
    """No rotation, one head, two eligible blocks: the first gets sigmoid(s0 - s1)."""
    q = np.zeros((1, 4, 1, 2))
    q[0, 3, 0] = [1.0, 0.0]
    k = np.array([[2.0, 0.0], [0.0, 1.0], [-1.0, 0.0], [3.0, 5.0]]).reshape(1, 4, 2)
    imp, _ = qsa.importance(q, k, r=2, rope_dims=0)
    s0, s1 = 1.0 / math.sqrt(2.0), 1.0 / math.sqrt(2.0)  # kbar0 = (1, .5), kbar1 = (1, 2.5)
    assert math.isclose(imp[0, 3, 0], 1.0 / (1.0 + math.exp(s1 - s0)), rel_tol=1e-14)
    q[0, 3, 0] = [0.0, 1.0]  # scores .5/sqrt2 and 2.5/sqrt2
    imp, _ = qsa.importance(q, k, r=2, rope_dims=0)
    assert math.isclose(imp[0, 3, 0], 1.0 / (1.0 + math.exp(2.0 / math.sqrt(2.0))), rel_tol=1e-14)
    # tokens 1 and 2 see only block 0 (token 2's own block is incomplete); token 0 sees none
    assert imp[0, 1, 0] == 1.0 and imp[0, 0].sum() == 0.0  # q = 0: all mass on block 0
    assert imp[0, 2, 1] == 0.0


def test_importance_zero_query_is_uniform():
    q, k = small_case(5)
    q[:, 20] = 0.0
    imp, elig = qsa.importance(q, k, r=4, rope_dims=8)
    n = elig[20].sum()
    assert np.allclose(imp[:, 20, elig[20]], 4.0 / n, atol=1e-15)


def test_pooling_comes_before_rotation():
    """A block has one position, so reordering keys inside a block changes nothing; rotating
    each token before averaging would depend on the order."""
    q, k = small_case(6, T=24)
    imp, _ = qsa.importance(q, k, r=4, rope_dims=16)
    k2 = k.copy()
    for j in range(6):
        k2[:, 4 * j:4 * j + 4] = k2[:, 4 * j:4 * j + 4][:, ::-1]
    imp2, _ = qsa.importance(q, k2, r=4, rope_dims=16)
    assert np.allclose(imp, imp2, atol=1e-13)


def test_block_position_is_its_first_token():
    """r = 2: block j sits at position 2j (its first token), so against the query at t = 5 the
    score of block j is a product at distance 5 - 2j; a last-token or mean position fails."""
    g = rng(7)
    d = 8
    k = g.standard_normal((1, 6, d))
    q = g.standard_normal((1, 6, 1, d))
    imp, _ = qsa.importance(q, k, r=2, rope_dims=d, base=10.0)
    kbar = [(k[0, 2 * j] + k[0, 2 * j + 1]) / 2 for j in range(3)]
    # relative form: rotate only the query, by the distance
    s = np.array([qsa.rope(q[0, 5, 0], float(5 - 2 * j), d, 10.0) @ kbar[j]
                  for j in range(3)]) / math.sqrt(d)
    p = np.exp(s - s.max())
    assert np.allclose(imp[0, 5], p / p.sum(), atol=1e-13)


def test_importance_is_causal():
    q, k = small_case(8)
    imp, elig = qsa.importance(q, k, r=4, rope_dims=8)
    t = 21  # eligible blocks 0..4 (tokens 0..19); tokens 20.. must not matter
    k2 = k.copy()
    k2[:, 20:] = rng(9).standard_normal(k2[:, 20:].shape) * 10
    imp2, _ = qsa.importance(q, k2, r=4, rope_dims=8)
    assert np.array_equal(imp[:, t], imp2[:, t])
    assert not np.allclose(imp[:, 36], imp2[:, 36])


def test_scale_zero_is_uniform():
    q, k = small_case(10)
    imp, elig = qsa.importance(q, k, r=4, rope_dims=8, scale=0.0)
    n = elig.sum(axis=1)
    for t in range(37):
        if n[t]:
            assert np.allclose(imp[:, t, elig[t]], 4.0 / n[t], atol=1e-15)


# ---- selection
def rank_select(imp_row, elig_row, nsel):
    """Independent definition: block j is kept iff fewer than nsel eligible blocks beat it,
    where i beats j if its importance is larger, or equal with a smaller index."""
    keep = []
    cand = [j for j in range(len(imp_row)) if elig_row[j]]
    for j in cand:
        better = sum(1 for i in cand if imp_row[i] > imp_row[j] or
                     (imp_row[i] == imp_row[j] and i < j))
        if better < nsel:
            keep.append(j)
    return keep


@pytest.mark.parametrize("nsel", [1, 3, 5, 100])
def test_select_matches_rank_definition(nsel):
    q, k = small_case(11, T=45)
    imp, elig = qsa.importance(q, k, r=2, rope_dims=16)
    sel = qsa.select(imp, elig, nsel)
    for b in range(2):
        for t in range(45):
            want = rank_select(imp[b, t], elig[t], nsel)
            got = [j for j in sel[b, t] if j >= 0]
            assert got == want
            assert (sel[b, t, len(want):] == -1).all()


def test_select_ties_go_to_the_lower_index():
    """Identical pooled keys without rotation give exactly equal importance."""
    q, k = small_case(12, B=1, T=32, d=8)
    k[0, :] = k[0, :4].mean(axis=0)  # every block pools to the same key
    imp, elig = qsa.importance(q, k, r=4, rope_dims=0)
    sel = qsa.select(imp, elig, 3)
    assert sel[0, 31].tolist() == [0, 1, 2]
    q[:] = 0.0
    imp, elig = qsa.importance(q, k, r=4, rope_dims=8)
    sel = qsa.select(imp, elig, 5)
    assert sel[0, 31].tolist() == [0, 1, 2, 3, 4]
    assert sel[0, 10].tolist() == [0, 1, -1, -1, -1]  # two eligible blocks only
    assert sel[0, 2].tolist() == [-1] * 5


def test_expand_tokens():
    sel = np.array([[[0, 2, -1]]])
    tok = qsa.expand_tokens(sel, r=4, T=11)
    assert tok[0, 0].tolist() == [0, 1, 2, 3, 8, 9, 10, -1, -1, -1, -1, -1]


def test_full_indexer_shapes():
    q, k = small_case(13, B=1, T=40, d=16)
    sel, imp = qsa.qsa_index(q, k, r=4, budget_tokens=12, rope_dims=8)
    assert sel.shape == (1, 40, 3) and imp.shape == (1, 40, 10)


def test_importance_of_selected_rows():
    q, k = small_case(14, T=41)
    full, elig = qsa.importance(q, k, r=4, rope_dims=8)
    rows = [40, 3, 17, 0]
    part, pe = qsa.importance(q, k, r=4, rope_dims=8, rows=rows)
    assert np.allclose(part, full[:, rows], atol=1e-15) and np.array_equal(pe, elig[rows])
