"""Pins of oracle/select.py (block scores, TopK / TopP selection, Variable Block expansion)
and of the variable-block predicate in oracle/masks.py, against facts fixed by the
definitions: a hand-computed example, bilinearity, closed forms for equal scores,
dominance and mass conditions, and brute force over every (query, key) pair."""
import math

import numpy as np
import pytest

from masked_long_context_tiled_amd.inputs import (MaskSpec, attention_inputs, bf16_bits_to_f64,
                                                  block_sparse_keep, variable_block_grid, variable_block_keep)
from oracle.masks import mask_block
from oracle.select import (block_scores, expand_variable_blocks, select_topk, select_topp, selection_order,
                           softmax_row)


def test_block_scores_hand_example():
    # T = 4, blocks of 2, d = 2, scale 1: block means of Q are (2, 0), (0, 3), of K (1, 2), (3, 0)
    q = np.array([[1, 0], [3, 0], [0, 2], [0, 4]], dtype=np.float64)[:, None, :]
    k = np.array([[1, 1], [1, 3], [2, 0], [4, 0]], dtype=np.float64)[:, None, :]
    s = block_scores(q, k, 2, scale=1.0)
    assert s.shape == (1, 2, 2)
    assert np.array_equal(s[0], np.array([[2.0, 6.0], [6.0, 0.0]]))


@pytest.mark.parametrize("T,b", [(37, 8), (64, 16), (50, 64)])
def test_block_scores_are_block_means_of_scores(T, b):
    rng = np.random.default_rng(T + b)
    Hq, Hk, d = 4, 2, 16
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((T, Hk, d))
    s = block_scores(q, k, b)
    nb = -(-T // b)
    for h in range(Hq):
        full = (q[:, h, :] @ k[:, h // 2, :].T) / math.sqrt(d)
        for qb in range(nb):
            for kb in range(nb):
                blk = full[qb * b:(qb + 1) * b, kb * b:(kb + 1) * b]
                assert abs(blk.mean() - s[h, qb, kb]) < 1e-12


def _rand_scores(seed, Hq=3, nb=11):
    return np.random.default_rng(seed).standard_normal((Hq, nb, nb))


@pytest.mark.parametrize("k", [1, 3, 6, 11, 20])
@pytest.mark.parametrize("diag", [True, False])
def test_topk_counts_and_dominance(k, diag):
    s = _rand_scores(k)
    keep = select_topk(s, k, diag)
    nb = s.shape[2]
    assert (keep.sum(axis=2) == min(k, nb)).all()
    for h in range(s.shape[0]):
        for qb in range(nb):
            if diag:
                assert keep[h, qb, qb] == 1
            others = np.array([kb for kb in range(nb) if not (diag and kb == qb)])
            kept = [s[h, qb, c] for c in others if keep[h, qb, c]]
            dropped = [s[h, qb, c] for c in others if not keep[h, qb, c]]
            if kept and dropped:
                assert min(kept) >= max(dropped)


def test_topk_equal_scores_keep_lowest_indices():
    nb, k = 9, 4
    s = np.zeros((2, nb, nb))
    keep = select_topk(s, k, True)
    for qb in range(nb):
        want = {qb} | set([c for c in range(nb) if c != qb][:k - 1])
        assert set(np.flatnonzero(keep[0, qb])) == want
    keep = select_topk(s, k, False)
    assert (keep[:, :, :k] == 1).all() and (keep[:, :, k:] == 0).all()


@pytest.mark.parametrize("p,nb", [(0.35, 10), (0.55, 9), (0.9, 7), (0.01, 12)])
def test_topp_equal_scores_closed_form(p, nb):
    # every block has mass 1/nb, so the shortest prefix reaching p has ceil(p nb) blocks
    assert abs(p * nb - round(p * nb)) > 1e-6
    s = np.zeros((1, nb, nb))
    keep = select_topp(s, p, False)
    assert (keep.sum(axis=2) == math.ceil(p * nb)).all()
    assert (keep[0, :, :math.ceil(p * nb)] == 1).all()
    keep = select_topp(s, p, True)
    assert (keep.sum(axis=2) == math.ceil(p * nb)).all()
    assert all(keep[0, qb, qb] == 1 for qb in range(nb))


@pytest.mark.parametrize("p", [0.2, 0.5, 0.8, 0.99])
@pytest.mark.parametrize("diag", [True, False])
def test_topp_mass_and_prefix(p, diag):
    s = 3.0 * _rand_scores(int(100 * p))
    keep = select_topp(s, p, diag)
    nb = s.shape[2]
    for h in range(s.shape[0]):
        for qb in range(nb):
            prob = softmax_row(s[h, qb])
            order = selection_order(s[h, qb], qb, diag)
            n = int(keep[h, qb].sum())
            assert set(np.flatnonzero(keep[h, qb])) == set(order[:n])   # a prefix of the order
            mass = prob[keep[h, qb] == 1].sum()
            assert mass >= p - 1e-12
            assert mass - prob[order[n - 1]] < p                          # shortest such prefix
            if diag:
                assert keep[h, qb, qb] == 1


def test_topp_one_keeps_everything_and_tiny_p_keeps_the_first():
    s = _rand_scores(5)
    assert (select_topp(s, 1.0, False) == 1).all()
    keep = select_topp(s, 1e-9, False)
    assert (keep.sum(axis=2) == 1).all()
    assert (np.argmax(keep, axis=2) == np.argmax(s, axis=2)).all()
    keep = select_topp(s, 1e-9, True)
    assert (keep.sum(axis=2) == 1).all()
    assert all(keep[h, qb, qb] for h in range(s.shape[0]) for qb in range(s.shape[1]))


def test_planted_block_is_selected():
    # all queries point along u; only the keys of block 5 share that direction
    T, b, d = 512, 64, 128
    x = attention_inputs(3, T, 2, 1)
    q = 0.05 * bf16_bits_to_f64(x["q"])
    k = 0.05 * bf16_bits_to_f64(x["k"])
    u = np.zeros(d)
    u[:8] = 1.0
    q += u
    k[5 * b:6 * b, 0, :] += 2.0 * u
    s = block_scores(q, k, b)
    keep = select_topk(s, 1, False)
    assert (np.argmax(keep, axis=2) == 5).all()


def test_variable_block_with_equal_sizes_is_uniform_block():
    T, b, Hq = 300, 64, 2
    off = tuple(list(range(0, T, b)) + [T])
    keep = block_sparse_keep(4, Hq, len(off) - 1, len(off) - 1)
    var = MaskSpec("variable_block", row_offsets=off, col_offsets=off)
    uni = MaskSpec("block_sparse", sparse_block=b)
    for h in range(Hq):
        assert np.array_equal(mask_block(var, T, range(T), range(T), h, keep),
                              mask_block(uni, T, range(T), range(T), h, keep))


@pytest.mark.parametrize("seed", [0, 1])
def test_variable_block_brute_force_and_expansion(seed):
    T, Hq = 1000, 3
    ro = variable_block_grid(seed, T)
    co = variable_block_grid(seed + 10, T)
    keep = variable_block_keep(seed, Hq, ro, co)
    spec = MaskSpec("variable_block", row_offsets=ro, col_offsets=co)
    k64 = expand_variable_blocks(keep, ro, co)
    uni = MaskSpec("block_sparse", sparse_block=64)
    for h in range(Hq):
        m = mask_block(spec, T, range(T), range(T), h, keep)
        # brute force: the block pair of every (i, j) from scanning the edges
        rb = np.array([max(r for r in range(len(ro) - 1) if ro[r] <= i) for i in range(T)])
        cb = np.array([max(c for c in range(len(co) - 1) if co[c] <= j) for j in range(T)])
        assert np.array_equal(m, keep[h][rb[:, None], cb[None, :]].astype(bool))
        assert np.array_equal(m, mask_block(uni, T, range(T), range(T), h, k64))
        # visible pairs = sum over kept block pairs of their areas
        area = np.outer(np.diff(ro), np.diff(co))
        assert m.sum() == int((area * keep[h]).sum())


def test_variable_block_generators():
    T = 4096
    ro = variable_block_grid(2, T)
    assert ro[0] == 0 and ro[-1] == T and all(0 < b - a <= 512 for a, b in zip(ro, ro[1:]))
    assert all(x % 64 == 0 for x in ro[:-1])
    keep = variable_block_keep(2, 2, ro, ro)
    size = np.diff(ro)
    covered = (keep * size[None, None, :]).sum(axis=2)
    assert (2 * covered >= T).all() and (keep.sum(axis=2) >= 1).all()
