"""Pins of the oracle's context tower and multi-block generation.

The causal attention against torch's causal scaled-dot-product attention (and an explicit
mask when a prefix precedes the block), causality of the whole context tower (later
tokens never change earlier K/V), the first layer's K/V in closed form, and the
multi-block loop reduced to the one-block loop over an explicitly extended prefix.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import OracleContextTower, oracle_generate, oracle_generate_blocks, rmsnorm, round_bf16
from oracle.denoise import joint_attention
from synth import draw_tower
from tests.helpers import inputs, make_oracle, mini_workload, oracle_weights


def _ctx(w):
    tw = draw_tower(w, context=True)
    W = oracle_weights(tw)
    return OracleContextTower(W, H=w.H, Hkv=w.Hkv, hd=w.hd, eps=w.rms_eps), W


@pytest.mark.parametrize("H,Hkv", [(4, 4), (4, 2)])
def test_causal_attention_matches_torch_without_prefix(H, Hkv):
    rng = np.random.default_rng(0)
    B, hd = 6, 8
    q = rng.normal(size=(B, H, hd))
    k = rng.normal(size=(B, Hkv, hd))
    v = rng.normal(size=(B, Hkv, hd))
    o = joint_attention(q, np.zeros((0, Hkv, hd)), np.zeros((0, Hkv, hd)), k, v, causal=True)
    G = H // Hkv
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(np.repeat(k, G, axis=1)).permute(1, 0, 2)
    tv = torch.from_numpy(np.repeat(v, G, axis=1)).permute(1, 0, 2)
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_causal_attention_with_prefix_matches_an_explicit_mask():
    rng = np.random.default_rng(1)
    P, B, H, hd = 5, 4, 2, 8
    q = rng.normal(size=(B, H, hd))
    kp, vp = rng.normal(size=(P, H, hd)), rng.normal(size=(P, H, hd))
    kb, vb = rng.normal(size=(B, H, hd)), rng.normal(size=(B, H, hd))
    o = joint_attention(q, kp, vp, kb, vb, causal=True)
    mask = np.ones((B, P + B), bool)
    mask[:, P:] = np.tril(np.ones((B, B), bool))
    tk = torch.from_numpy(np.concatenate([kp, kb])).permute(1, 0, 2)
    tv = torch.from_numpy(np.concatenate([vp, vb])).permute(1, 0, 2)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q).permute(1, 0, 2), tk, tv,
                                         attn_mask=torch.from_numpy(mask)).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    # the last block query sees everything: equal to the unmasked attention of that row
    full = joint_attention(q, kp, vp, kb, vb, causal=False)
    np.testing.assert_allclose(o[-1], full[-1], rtol=1e-12, atol=1e-12)


def test_context_tower_is_causal():
    """Changing tokens after position p leaves every layer's k/v at positions <= p unchanged."""
    w = mini_workload()
    ctx, _ = _ctx(w)
    plens, tau, kv = inputs(w)
    rng = np.random.default_rng(2)
    tok = rng.integers(0, w.V, size=(w.n, w.B))
    base = ctx.block_kv(tok, kv, range(w.n))
    p = 3
    tok2 = tok.copy()
    tok2[:, p + 1:] = rng.integers(0, w.V, size=(w.n, w.B - p - 1))
    alt = ctx.block_kv(tok2, kv, range(w.n))
    for (k, v), (k2, v2) in zip(base, alt):
        np.testing.assert_array_equal(k[:, :p + 1], k2[:, :p + 1])
        np.testing.assert_array_equal(v[:, :p + 1], v2[:, :p + 1])
    assert not np.allclose(base[-1][0][:, p + 1:], alt[-1][0][:, p + 1:])


def test_context_tower_first_layer_kv_closed_form():
    """Layer 0: k = rmsnorm(E[tok]) Wk^T, no position term, independent of the prefix."""
    w = mini_workload()
    ctx, W = _ctx(w)
    plens, tau, kv = inputs(w)
    tok = np.random.default_rng(3).integers(0, w.V, size=(w.n, w.B))
    k0, v0 = ctx.block_kv(tok, kv, range(w.n))[0]
    h = rmsnorm(W["tok_emb"][tok].astype(np.float64), W["attn_norm"][0].astype(np.float64), w.rms_eps)
    np.testing.assert_allclose(k0, (h @ W["wk"][0].astype(np.float64).T).reshape(k0.shape), rtol=1e-12)
    np.testing.assert_allclose(v0, (h @ W["wv"][0].astype(np.float64).T).reshape(v0.shape), rtol=1e-12)


def test_multi_block_reduces_to_the_one_block_loop():
    """Block 1 equals the one-block loop; block 2 equals the one-block loop over the prefix
    extended by the context tower's (bf16-rounded) K/V of block 1."""
    w = mini_workload()
    orc, _ = make_oracle(w)
    ctx, _ = _ctx(w)
    plens, tau, kv = inputs(w)
    toks, cst, steps = oracle_generate_blocks(orc, ctx, 2, w.n, w.B, tau, 0.8, kv, cache_bf16=True)
    t1, c1, s1, _ = oracle_generate(orc, w.n, w.B, tau, 0.8, kv, keep_trace=False)
    assert np.array_equal(toks[0], t1) and np.array_equal(cst[0], c1) and np.array_equal(steps[0], s1)
    kvs = ctx.block_kv(t1, kv, range(w.n))

    def kv2(l, s):
        K, V = kv(l, s)
        return (np.concatenate([K, round_bf16(kvs[l][0][s])]), np.concatenate([V, round_bf16(kvs[l][1][s])]))

    t2, c2, s2, _ = oracle_generate(orc, w.n, w.B, tau, 0.8, kv2, keep_trace=False)
    assert np.array_equal(toks[1], t2) and np.array_equal(cst[1], c2) and np.array_equal(steps[1], s2)
    assert not np.array_equal(toks[0], toks[1])


def _ctx_ar(w):
    tw = draw_tower(w, context=True, ar_head=True)
    W = oracle_weights(tw)
    return OracleContextTower(W, H=w.H, Hkv=w.Hkv, hd=w.hd, eps=w.rms_eps), W


def test_ar_step_without_prefix_attends_only_to_itself():
    """P = 0: one key, softmax weight 1, so every layer's attention output is the token's
    own value vector; the whole step is then a closed form of the MLP tower."""
    from oracle.denoise import gelu
    w = mini_workload(L=1)
    ctx, W = _ctx_ar(w)
    f64 = lambda a: np.asarray(a, np.float64)  # noqa: E731
    empty = lambda l, s: (np.zeros((0, w.Hkv, w.hd)), np.zeros((0, w.Hkv, w.hd)))  # noqa: E731
    tok = np.array([3, 7])
    kvs, z = ctx.ar_step(tok, empty, [0, 1])
    x = f64(W["tok_emb"][tok])
    h = rmsnorm(x, f64(W["attn_norm"][0]), w.rms_eps)
    v = (h @ f64(W["wv"][0]).T).reshape(2, w.Hkv, w.hd)
    o = np.repeat(v, w.H // w.Hkv, axis=1).reshape(2, -1)
    x = x + o @ f64(W["wo"][0]).T
    x = x + gelu(rmsnorm(x, f64(W["mlp_norm"][0]), w.rms_eps) @ f64(W["w1"][0]).T) @ f64(W["w2"][0]).T
    zc = rmsnorm(x, f64(W["final_norm"]), w.rms_eps) @ f64(W["lm_head"]).T
    np.testing.assert_allclose(z, zc, rtol=1e-12, atol=1e-12)


def test_ar_step_kv_equals_one_token_block_kv():
    """The K/V an AR step appends are the context tower's K/V of a one-token block."""
    w = mini_workload()
    ctx, _ = _ctx_ar(w)
    plens, tau, kv = inputs(w)
    tok = np.array([5, 11])
    kvs, _ = ctx.ar_step(tok, kv, range(w.n))
    ref = ctx.block_kv(tok[:, None], kv, range(w.n))
    for (k, v), (kr, vr) in zip(kvs, ref):
        np.testing.assert_array_equal(k, kr)
        np.testing.assert_array_equal(v, vr)


def test_ar_decode_is_greedy_and_appends():
    """Each decoded token is the argmax of the step's logits given all earlier appends."""
    from oracle import oracle_ar_decode
    w = mini_workload()
    ctx, _ = _ctx_ar(w)
    plens, tau, kv = inputs(w)
    first = np.array([1, 2])
    toks = oracle_ar_decode(ctx, first, 3, kv, cache_bf16=False)
    kvs0, z0 = ctx.ar_step(first, kv, range(w.n))
    assert np.array_equal(toks[:, 0], np.argmax(z0.astype(np.float32), axis=1))

    def kv1(l, s):
        K, V = kv(l, s)
        return np.concatenate([K, kvs0[l][0][s]]), np.concatenate([V, kvs0[l][1][s]])

    _, z1 = ctx.ar_step(toks[:, 0], kv1, range(w.n))
    assert np.array_equal(toks[:, 1], np.argmax(z1.astype(np.float32), axis=1))
