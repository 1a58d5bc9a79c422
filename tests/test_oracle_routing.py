"""Pins of top-k routing and the group-by-expert permutation: brute force,
ties, softmax against float64, permutation invariants."""
import numpy as np
import pytest

from oracle import moe


def _brute_topk(logits, k):
    T, E = logits.shape
    out = []
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))
        out.append(order[:k])
    return np.array(out, dtype=np.int32)


@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (64, 384, 6), (5, 6, 6), (3, 1, 1)])
def test_topk_brute_force(T, E, k):
    logits = np.random.default_rng(T + E).standard_normal((T, E)).astype(np.float32)
    ids, w = moe.route_topk(logits, k)
    assert np.array_equal(ids, _brute_topk(logits, k))


def test_topk_ties_go_to_lower_id():
    logits = np.zeros((4, 10), dtype=np.float32)
    logits[1, [3, 7]] = 1.0
    logits[2] = np.float32(0.5)
    logits[3, 9] = -0.0
    ids, w = moe.route_topk(logits, 3)
    assert ids[0].tolist() == [0, 1, 2]
    assert ids[1].tolist() == [3, 7, 0]
    assert ids[2].tolist() == [0, 1, 2]
    assert ids[3].tolist() == [0, 1, 2]          # -0.0 ties with +0.0
    assert np.array_equal(w[0], np.full(3, np.float32(1) / np.float32(3), dtype=np.float32))


def test_weights_are_softmax_of_selected_logits():
    rng = np.random.default_rng(1)
    logits = (rng.standard_normal((200, 384)) * 3).astype(np.float32)
    ids, w = moe.route_topk(logits, 6)
    sel = np.take_along_axis(logits, ids, 1).astype(np.float64)
    ref = np.exp(sel - sel[:, :1])
    ref /= ref.sum(1, keepdims=True)
    assert np.allclose(w, ref, rtol=4 * 2.0 ** -24 * 6, atol=1e-30)
    assert np.abs(w.astype(np.float64).sum(1) - 1).max() <= 8 * 2.0 ** -24
    assert (np.diff(w, axis=1) <= 0).all()       # slots are in descending order


@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (256, 384, 6), (7, 50, 3)])
def test_permutation_invariants(T, E, k):
    logits = np.random.default_rng(T).standard_normal((T, E)).astype(np.float32)
    ids, _ = moe.route_topk(logits, k)
    off, sorted_ids, inv = moe.permute(ids, E)
    assert off[0] == 0 and off[-1] == T * k
    assert np.array_equal(np.diff(off), np.bincount(ids.reshape(-1), minlength=E))
    seen = np.zeros(T * k, dtype=int)
    for t in range(T):
        for j in range(k):
            p = inv[t, j]
            seen[p] += 1
            assert sorted_ids[p] == t
            e = ids[t, j]
            assert off[e] <= p < off[e + 1]
    assert (seen == 1).all()
    # inside an expert, rows are ascending in flat index t*k+j
    flat_of_row = np.empty(T * k, dtype=np.int64)
    flat_of_row[inv.reshape(-1)] = np.arange(T * k)
    for e in range(E):
        seg = flat_of_row[off[e]:off[e + 1]]
        assert (np.diff(seg) > 0).all()


def test_permutation_brute_force_small():
    ids = np.array([[2, 0], [0, 1], [2, 1], [1, 0]], dtype=np.int32)
    off, sorted_ids, inv = moe.permute(ids, 4)
    assert off.tolist() == [0, 3, 6, 8, 8]
    # expert 0: (0,1),(1,0),(3,1); expert 1: (1,1),(2,1),(3,0); expert 2: (0,0),(2,0)
    assert sorted_ids.tolist() == [0, 1, 3, 1, 2, 3, 0, 2]
    assert inv.tolist() == [[6, 0], [1, 3], [7, 4], [5, 2]]
