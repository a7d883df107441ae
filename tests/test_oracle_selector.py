"""Pins of the oracle's candidate selector ("DFlash vs DFlash 2", "The candidate
selector": S_t(a, b) = U_t(b) + <A(a) * H(h_t), B(b)>, then one walk from the
anchor).  Each test fixes the answer by construction, not by re-evaluating the
score formula."""
import numpy as np
import pytest

import oracle


def _rand_case(seed, B=3, G=5, k=6, V=40, r=8):
    rng = np.random.default_rng(seed)
    cand = np.stack([np.stack([rng.permutation(V)[:k] for _ in range(G)]) for _ in range(B)])
    return (cand, rng.normal(size=(B, G, k)), rng.normal(size=(V, r)), rng.normal(size=(V, r)),
            rng.normal(size=(B, G, r)), rng.integers(0, V, B))


def test_zero_gate_walks_the_top1_of_each_position():
    cand, U, ea, eb, g, anc = _rand_case(0)
    out = oracle.select_path(cand, U, ea, eb, np.zeros_like(g), anc)
    top1 = np.take_along_axis(cand, U.argmax(axis=2)[..., None], axis=2)[..., 0]
    assert np.array_equal(out["path"], top1)
    assert np.allclose(out["score"], U.max(axis=2), rtol=0, atol=0)


def test_candidate_order_does_not_matter():
    cand, U, ea, eb, g, anc = _rand_case(1)
    ref = oracle.select_path(cand, U, ea, eb, g, anc)
    rng = np.random.default_rng(2)
    perm = np.stack([np.stack([rng.permutation(cand.shape[2]) for _ in range(cand.shape[1])])
                     for _ in range(cand.shape[0])])
    out = oracle.select_path(np.take_along_axis(cand, perm, 2), np.take_along_axis(U, perm, 2),
                             ea, eb, g, anc)
    assert np.array_equal(out["path"], ref["path"])
    assert np.allclose(out["score"], ref["score"], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("G", [1, 4, 8])
def test_planted_chain_is_followed_only_through_the_position_gate(G):
    """Chain tokens c_0 (anchor), c_1..c_G with A(c_t) = e_t, B(c_{t+1}) = 50 e_t
    and gate_t = e_t: the pair (c_t -> c_{t+1}) gains 50 at position t and nowhere
    else; U ranks the chain token last at every position.  A walk that used the
    wrong predecessor, gate row or embedding table would fall back to U's top-1."""
    V, r, k = 64, G + 1, 5
    rng = np.random.default_rng(G)
    chain = rng.permutation(V)[:G + 1]
    ea = np.zeros((V, r))
    eb = np.zeros((V, r))
    for t in range(G):
        ea[chain[t], t] = 1.0
        eb[chain[t + 1], t] = 50.0
    gate = np.zeros((1, G, r))
    for t in range(G):
        gate[0, t, t] = 1.0
    others = [v for v in range(V) if v not in set(chain.tolist())]
    cand = np.zeros((1, G, k), dtype=np.int64)
    U = np.zeros((1, G, k))
    for t in range(G):
        cand[0, t] = [others[(t * 7 + j) % len(others)] for j in range(k - 1)] + [chain[t + 1]]
        U[0, t] = np.linspace(3.0, 1.0, k)  # the chain token (listed last) has the lowest U
    out = oracle.select_path(cand, U, ea, eb, gate, [chain[0]])
    assert out["path"][0].tolist() == chain[1:].tolist()
    assert np.allclose(out["score"][0], 1.0 + 50.0)
    # a gate that is one position off removes every bonus
    shifted = np.roll(gate, 1, axis=1) if G > 1 else np.zeros_like(gate)
    off = oracle.select_path(cand, U, ea, eb, shifted, [chain[0]])
    assert off["path"][0].tolist() == cand[0, :, 0].tolist()


def test_walk_is_greedy_not_best_path():
    """Position 0: x (U = 1.0) beats y (U = 0.9); position 1 pays 10 only after y.
    The best two-step path is y -> u (10.9) but the greedy walk takes x and then
    the first-listed of two equal scores."""
    V, r = 6, 1
    a0, x, y, u, w = 0, 1, 2, 3, 4
    ea = np.zeros((V, r))
    eb = np.zeros((V, r))
    ea[y, 0] = 1.0
    eb[u, 0] = 10.0
    cand = np.array([[[x, y], [u, w]]])
    U = np.array([[[1.0, 0.9], [0.0, 0.0]]])
    gate = np.ones((1, 2, r))
    out = oracle.select_path(cand, U, ea, eb, gate, [a0])
    assert out["path"][0].tolist() == [x, u]
    assert out["score"][0].tolist() == [1.0, 0.0]
    # with x's lead removed the walk goes through y and collects the bonus
    U2 = np.array([[[0.8, 0.9], [0.0, 0.0]]])
    out2 = oracle.select_path(cand, U2, ea, eb, gate, [a0])
    assert out2["path"][0].tolist() == [y, u]
    assert out2["score"][0].tolist() == [0.9, 10.0]


def test_ties_go_to_the_first_listed_candidate():
    cand = np.array([[[5, 2, 9]]])
    U = np.array([[[0.5, 0.5, 0.5]]])
    out = oracle.select_path(cand, U, np.zeros((10, 2)), np.zeros((10, 2)), np.zeros((1, 1, 2)), [1])
    assert out["path"][0, 0] == 5


def test_rejects_out_of_range_tokens():
    cand = np.array([[[5, 12]]])
    with pytest.raises(ValueError):
        oracle.select_path(cand, np.zeros((1, 1, 2)), np.zeros((10, 2)), np.zeros((10, 2)),
                           np.zeros((1, 1, 2)), [1])
