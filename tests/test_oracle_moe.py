"""Pins of the oracle's mixture-of-experts MLP (oracle.moe_route, oracle.moe_ffn).

The pages give counts only (dzen, section "Что нового": 6 of 128 experts plus 2 shared
per token), no worked example, so the pins are reductions to the dense tower (already
pinned elsewhere), closed forms on crafted router scores and experts, tie and precision
cases of the routing decision, and equivariance under relabelling the experts.
"""
import numpy as np
import pytest

from oracle import OracleTower, moe_ffn, moe_route
from tests.helpers import inputs, make_oracle, mini_workload


def _dense_and_moe(moe_of_w):
    """The mini tower dense, and the same tower with its MLPs replaced by moe_of_w(W, l)."""
    w = mini_workload()
    dense, W = make_oracle(w)
    layers = [moe_of_w(W, l) for l in range(w.L)]
    moe = dict(top_k=layers[0]["top_k"], router=[m["router"] for m in layers], w1=[m["w1"] for m in layers],
               w2=[m["w2"] for m in layers], sw1=[m["sw1"] for m in layers], sw2=[m["sw2"] for m in layers])
    Wm = dict(W)
    Wm["moe"] = moe
    tower = OracleTower(Wm, H=w.H, Hkv=w.Hkv, hd=w.hd, eps=w.rms_eps)
    plens, tau, kv = inputs(w)
    rng = np.random.default_rng(5)
    tok = rng.integers(0, w.V + 1, size=(w.n, w.B))
    return dense.hidden(tok, kv, range(w.n)), tower, tok, kv, w


def test_single_expert_top1_is_the_dense_mlp():
    """E = 1, top_k = 1, no shared expert: the gate is 1 and the MoE is the dense MLP."""
    ref, tower, tok, kv, w = _dense_and_moe(lambda W, l: dict(
        top_k=1, router=np.ones((1, W["w1"][l].shape[1])), w1=[W["w1"][l]], w2=[W["w2"][l]], sw1=[], sw2=[]))
    np.testing.assert_allclose(tower.hidden(tok, kv, range(w.n)), ref, rtol=0, atol=1e-12)


def test_shared_expert_alone_is_the_dense_mlp():
    """Routed experts that output zero (W2 = 0) plus one shared expert holding the dense
    weights: the shared expert enters with weight 1."""
    def mk(W, l):
        F, d = W["w1"][l].shape
        rng = np.random.default_rng(l)
        return dict(top_k=2, router=rng.standard_normal((4, d)), w1=[rng.standard_normal((8, d))] * 4,
                    w2=[np.zeros((d, 8))] * 4, sw1=[W["w1"][l]], sw2=[W["w2"][l]])
    ref, tower, tok, kv, w = _dense_and_moe(mk)
    np.testing.assert_allclose(tower.hidden(tok, kv, range(w.n)), ref, rtol=0, atol=1e-12)


def test_identical_experts_all_chosen_sum_to_the_dense_mlp():
    """Three identical experts, all chosen: the gates sum to 1, whatever the scores."""
    def mk(W, l):
        d = W["w1"][l].shape[1]
        rng = np.random.default_rng(10 + l)
        return dict(top_k=3, router=rng.standard_normal((3, d)), w1=[W["w1"][l]] * 3, w2=[W["w2"][l]] * 3,
                    sw1=[], sw2=[])
    ref, tower, tok, kv, w = _dense_and_moe(mk)
    np.testing.assert_allclose(tower.hidden(tok, kv, range(w.n)), ref, rtol=0, atol=1e-10)


def _scaled_identity_experts(scales, d):
    """Expert e maps a unit vector u to scales[e] * u: W1 = scales[e] * I, W2 = I, and
    gelu(a) = a to float64 precision for a >= 10 (1 - Phi(10) < 1e-23)."""
    return [np.eye(d) * s for s in scales], [np.eye(d)] * len(scales)


def test_route_and_gates_closed_form():
    """Rows are unit vectors, so row r's score for expert e is router[e][r].  Top-2 of
    row 0 scores (2, 0.5, 1, -1) is experts 0 then 2 with gates e/(1+e) and 1/(1+e)."""
    d = 4
    router = np.array([[2.0, 0.0, 1.0, 3.0],
                       [0.5, 0.0, 1.0, 2.0],
                       [1.0, 0.0, 1.0, 1.0],
                       [-1.0, 0.0, 1.0, 0.0]])   # [E = 4][d]; column r = scores of row r
    h2 = np.eye(d)
    w1, w2 = _scaled_identity_experts([10.0, 20.0, 30.0, 40.0], d)
    y, ex, gt, sc = moe_ffn(h2, router, w1, w2, [], [], top_k=2)
    np.testing.assert_array_equal(sc, router.T)
    g_hi, g_lo = np.e / (1 + np.e), 1 / (1 + np.e)
    # row 0: scores (2, .5, 1, -1) -> experts 0, 2
    assert ex[0].tolist() == [0, 2]
    np.testing.assert_allclose(gt[0], [g_hi, g_lo], rtol=1e-15)
    np.testing.assert_allclose(y[0], [10 * g_hi + 30 * g_lo, 0, 0, 0], rtol=1e-14, atol=1e-14)
    # row 1: all scores 0 -> the lowest ids 0, 1, equal gates
    assert ex[1].tolist() == [0, 1]
    np.testing.assert_allclose(y[1], [0, 0.5 * 10 + 0.5 * 20, 0, 0], rtol=1e-14, atol=1e-14)
    # row 2: scores (1, 1, 1, 1) -> 0, 1
    assert ex[2].tolist() == [0, 1]
    # row 3: scores (3, 2, 1, 0) -> 0, 1 with gates e/(1+e), 1/(1+e)
    assert ex[3].tolist() == [0, 1]
    np.testing.assert_allclose(y[3], [0, 0, 0, 10 * g_hi + 20 * g_lo], rtol=1e-14, atol=1e-14)


def test_shared_experts_add_with_weight_one_closed_form():
    d = 2
    router = np.array([[1.0, 0.0], [0.0, 1.0]])
    w1, w2 = _scaled_identity_experts([10.0, 20.0], d)
    sw1, sw2 = _scaled_identity_experts([50.0, 70.0], d)
    y, ex, gt, _ = moe_ffn(np.eye(d), router, w1, w2, sw1, sw2, top_k=1)
    assert ex[:, 0].tolist() == [0, 1]
    np.testing.assert_allclose(y, np.diag([10.0 + 120.0, 20.0 + 120.0]), rtol=1e-15)


def test_route_decides_in_float32():
    """Scores equal in float32 but not in float64 are a tie: the lowest id wins."""
    s = np.array([[1.0, 1.0 + 1e-12, 0.5], [1.0 + 1e-12, 1.0, 0.5], [0.5, 1.0, 1.0 + 1e-6]])
    ex, gt = moe_route(s, 1)
    assert ex[:, 0].tolist() == [0, 0, 2]
    np.testing.assert_allclose(gt, 1.0)
    ex2, gt2 = moe_route(s, 2)
    assert ex2.tolist() == [[0, 1], [0, 1], [2, 1]]
    np.testing.assert_allclose(gt2.sum(axis=1), 1.0, rtol=1e-15)


def test_route_rejects_bad_top_k():
    with pytest.raises(ValueError):
        moe_route(np.zeros((1, 4)), 0)
    with pytest.raises(ValueError):
        moe_route(np.zeros((1, 4)), 5)


def test_relabelling_experts_permutes_routes_and_keeps_outputs():
    """Expert e of one MoE is expert perm[e] of the other: routes map through perm and
    the outputs agree; an implementation that indexed experts by rank would not."""
    rng = np.random.default_rng(3)
    R, d, E, de, k = 12, 16, 8, 24, 3
    h2 = rng.standard_normal((R, d))
    router = rng.standard_normal((E, d))
    w1 = [rng.standard_normal((de, d)) * 0.3 for _ in range(E)]
    w2 = [rng.standard_normal((d, de)) * 0.3 for _ in range(E)]
    sw1, sw2 = [rng.standard_normal((de, d)) * 0.3], [rng.standard_normal((d, de)) * 0.3]
    perm = rng.permutation(E)
    inv = np.argsort(perm)
    y, ex, gt, _ = moe_ffn(h2, router, w1, w2, sw1, sw2, k)
    y2, ex2, gt2, _ = moe_ffn(h2, router[inv], [w1[i] for i in inv], [w2[i] for i in inv], sw1, sw2, k)
    np.testing.assert_array_equal(perm[ex], ex2)
    np.testing.assert_allclose(gt, gt2, rtol=1e-15)
    np.testing.assert_allclose(y, y2, rtol=1e-12, atol=1e-12)
    # a different choice of experts changes the output (the pin has teeth)
    y3, *_ = moe_ffn(h2, router, w1[::-1], w2[::-1], sw1, sw2, k)
    assert np.abs(y3 - y).max() > 1e-3


def test_gates_are_monotone_in_rank_and_sum_to_one():
    rng = np.random.default_rng(4)
    s = rng.standard_normal((50, 128))
    ex, gt = moe_route(s, 6)
    np.testing.assert_allclose(gt.sum(axis=1), 1.0, rtol=1e-14)
    assert (np.diff(gt, axis=1) <= 0).all()
    # the chosen experts are the six largest scores
    np.testing.assert_array_equal(np.sort(ex, axis=1), np.sort(np.argsort(-s, axis=1)[:, :6], axis=1))
