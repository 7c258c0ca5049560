"""Pins of the oracle's parts against library routines, closed forms and brute force."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import commit_rule, gelu, joint_attention, rmsnorm, round_bf16, vocab_reduce

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------- bf16 rounding

def test_round_bf16_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000)).astype(np.float32)
    ties = ((rng.integers(0, 1 << 7, 1000, dtype=np.uint32) << 16) | np.uint32(0x8000)
            | (rng.integers(0, 2, 1000, dtype=np.uint32) << 31) | np.uint32(0x40000000)).view(np.float32)
    sub = np.array([1e-40, -2.5e-39, 9.2e-41, 1.17e-38], dtype=np.float32)   # bf16 subnormals
    x = np.concatenate([x, ties, sub])
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(round_bf16(x.astype(np.float64)), ref)


def test_round_bf16_closed_forms():
    assert round_bf16(1.0) == 1.0
    assert round_bf16(1.0 + 2.0 ** -8) == 1.0            # tie -> even (1.0)
    assert round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6   # tie -> even (odd 1+2^-7 goes up)
    assert round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7   # past the tie
    assert round_bf16(-3.0) == -3.0 and round_bf16(0.0) == 0.0


# --------------------------------------------------------------------------- rmsnorm / gelu

def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 33))
    g = rng.standard_normal(33)
    ref = F.rms_norm(torch.from_numpy(x), (33,), weight=torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(rmsnorm(x, g, 1e-6), ref, rtol=1e-13, atol=1e-14)


def test_rmsnorm_constant_vector_closed_form():
    c = -0.37
    out = rmsnorm(np.full((1, 10), c), np.ones(10), 1e-6)
    np.testing.assert_allclose(out, c / math.sqrt(c * c + 1e-6), rtol=1e-14)


def test_gelu_matches_torch_exact_form():
    x = np.linspace(-8, 8, 4001)
    ref = F.gelu(torch.from_numpy(x), approximate="none").numpy()
    np.testing.assert_allclose(gelu(x), ref, rtol=1e-14, atol=1e-15)
    # the tanh approximation differs by more than 1e-4 somewhere: the form matters
    tanh = F.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.abs(gelu(x) - tanh).max() > 1e-4


def test_gelu_identities():
    x = np.linspace(-5, 5, 101)
    np.testing.assert_allclose(gelu(x) - gelu(-x), x, atol=1e-14)
    assert gelu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(gelu(np.array([1.0]))[0], 0.5 * (1 + math.erf(1 / math.sqrt(2))), rtol=1e-15)


# --------------------------------------------------------------------------- attention

def _rand_attn(rng, B, H, Hkv, hd, P):
    q = rng.standard_normal((B, H, hd))
    kp, vp = rng.standard_normal((P, Hkv, hd)), rng.standard_normal((P, Hkv, hd))
    kb, vb = rng.standard_normal((B, Hkv, hd)), rng.standard_normal((B, Hkv, hd))
    return q, kp, vp, kb, vb


@pytest.mark.parametrize("B,H,Hkv,hd,P", [(4, 2, 2, 8, 5), (3, 4, 2, 4, 0), (8, 6, 3, 16, 33), (2, 8, 1, 8, 1)])
def test_attention_matches_torch_sdpa(B, H, Hkv, hd, P):
    rng = np.random.default_rng(B * 100 + P)
    q, kp, vp, kb, vb = _rand_attn(rng, B, H, Hkv, hd, P)
    K = torch.from_numpy(np.concatenate([kp, kb], 0)).permute(1, 0, 2)[None]
    Vt = torch.from_numpy(np.concatenate([vp, vb], 0)).permute(1, 0, 2)[None]
    Q = torch.from_numpy(q).permute(1, 0, 2)[None]
    ref = F.scaled_dot_product_attention(Q, K, Vt, enable_gqa=True)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(joint_attention(q, kp, vp, kb, vb), ref, rtol=1e-12, atol=1e-13)


def test_attention_matches_brute_force_ragged_batch():
    """Dense score matrix over two sequences' padded keys, -inf on padding, explicit loops."""
    rng = np.random.default_rng(5)
    B, H, Hkv, hd = 3, 4, 2, 4
    plens = [0, 5]
    Pmax = max(plens)
    seqs = [_rand_attn(rng, B, H, Hkv, hd, P) for P in plens]
    for (q, kp, vp, kb, vb), P in zip(seqs, plens):
        # pad the prefix to Pmax; padding keys hold garbage and must be masked
        kpad = np.concatenate([kp, 1e3 * rng.standard_normal((Pmax - P, Hkv, hd))], 0)
        vpad = np.concatenate([vp, 1e3 * rng.standard_normal((Pmax - P, Hkv, hd))], 0)
        out = np.zeros((B, H, hd))
        for b, j in itertools.product(range(B), range(H)):
            g = j // (H // Hkv)
            keys = [kpad[t, g] for t in range(Pmax)] + [kb[t, g] for t in range(B)]
            vals = [vpad[t, g] for t in range(Pmax)] + [vb[t, g] for t in range(B)]
            valid = [t < P for t in range(Pmax)] + [True] * B
            sc = [float(np.dot(q[b, j], kk)) / math.sqrt(hd) if ok else -math.inf for kk, ok in zip(keys, valid)]
            mx = max(sc)
            w = [math.exp(s - mx) for s in sc]
            tot = sum(w)
            for t in range(len(keys)):
                out[b, j] += (w[t] / tot) * vals[t]
        np.testing.assert_allclose(joint_attention(q, kp, vp, kb, vb), out, rtol=1e-12, atol=1e-13)


def test_attention_no_prefix_is_bidirectional_self_attention():
    rng = np.random.default_rng(6)
    q, _, _, kb, vb = _rand_attn(rng, 5, 2, 2, 8, 0)
    empty = np.zeros((0, 2, 8))
    Q = torch.from_numpy(q).permute(1, 0, 2)
    K = torch.from_numpy(kb).permute(1, 0, 2)
    Vt = torch.from_numpy(vb).permute(1, 0, 2)
    bi = F.scaled_dot_product_attention(Q, K, Vt).permute(1, 0, 2).numpy()
    causal = F.scaled_dot_product_attention(Q, K, Vt, is_causal=True).permute(1, 0, 2).numpy()
    ours = joint_attention(q, empty, empty, kb, vb)
    np.testing.assert_allclose(ours, bi, rtol=1e-12, atol=1e-13)
    assert np.abs(ours - causal).max() > 1e-3


def test_attention_special_cases():
    rng = np.random.default_rng(7)
    hd = 8
    # a single key (P=0, B=1): output is that key's value row
    q, kb, vb = rng.standard_normal((1, 2, hd)), rng.standard_normal((1, 1, hd)), rng.standard_normal((1, 1, hd))
    e = np.zeros((0, 1, hd))
    np.testing.assert_allclose(joint_attention(q, e, e, kb, vb)[0, 1], vb[0, 0], rtol=1e-14)
    # identical keys: output is the mean of the value rows
    kp = np.repeat(rng.standard_normal((1, 1, hd)), 6, axis=0)
    vp = rng.standard_normal((6, 1, hd))
    kb2 = kp[:2].copy()
    vb2 = rng.standard_normal((2, 1, hd))
    q2 = rng.standard_normal((2, 1, hd))
    out = joint_attention(q2, kp, vp, kb2, vb2)
    np.testing.assert_allclose(out[0, 0], np.concatenate([vp, vb2])[:, 0].mean(0), rtol=1e-12)
    # permuting prefix tokens leaves the output unchanged (no positional mask over the prefix)
    q3, kp3, vp3, kb3, vb3 = _rand_attn(rng, 4, 4, 2, hd, 9)
    perm = rng.permutation(9)
    np.testing.assert_allclose(joint_attention(q3, kp3[perm], vp3[perm], kb3, vb3),
                               joint_attention(q3, kp3, vp3, kb3, vb3), rtol=1e-12)


# --------------------------------------------------------------------------- vocab reduction

def test_vocab_reduce_matches_torch_softmax_and_argmax():
    rng = np.random.default_rng(8)
    z = rng.standard_normal((6, 1000))
    tau = np.array([1.0, 2.5, 10.0, 33.0, 64.0, 1.5])
    conf, arg, gap = vocab_reduce(z, tau)
    p = torch.softmax(torch.from_numpy(tau[:, None] * z), dim=1)
    np.testing.assert_allclose(conf, p.max(1).values.numpy(), rtol=1e-13)
    np.testing.assert_allclose(p.sum(1).numpy(), 1.0, atol=1e-12)
    assert np.array_equal(arg, torch.argmax(torch.from_numpy((tau[:, None] * z).astype(np.float32)), 1).numpy())
    top2 = torch.topk(p, 2, dim=1).values.numpy()
    np.testing.assert_allclose(gap, top2[:, 0] - top2[:, 1], rtol=1e-10, atol=1e-15)
    assert (conf >= 1 / 1000).all() and (conf <= 1).all()


def test_vocab_reduce_zero_head_and_ties():
    conf, arg, gap = vocab_reduce(np.zeros((3, 97)), np.array([1.0, 7.0, 64.0]))
    assert np.all(conf == 1.0 / 97) and np.all(arg == 0) and np.all(gap == 0)
    z = np.array([[0.5, 2.0, 2.0, -1.0]])
    assert vocab_reduce(z, np.array([3.0]))[1][0] == 1     # lowest id among equal maxima


def test_vocab_reduce_tau_invariance_and_monotonicity():
    rng = np.random.default_rng(9)
    z = rng.standard_normal((1, 500))
    taus = [1.0, 2.0, 4.0, 16.0, 64.0]
    res = [vocab_reduce(z, np.array([t])) for t in taus]
    assert len({int(r[1][0]) for r in res}) == 1
    confs = [float(r[0][0]) for r in res]
    assert all(a <= b for a, b in zip(confs, confs[1:]))


def test_vocab_reduce_golden():
    with open(os.path.join(GOLDEN, "vocab_reduce_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        conf, arg, gap = vocab_reduce(np.array([c["z"]], dtype=np.float64), np.array([c["tau"]]))
        assert arg[0] == c["arg"], c
        np.testing.assert_allclose(conf[0], c["conf"], rtol=1e-12)
        np.testing.assert_allclose(gap[0], c["gap"], rtol=1e-12, atol=1e-15)


# --------------------------------------------------------------------------- commit rule

def test_commit_rule_golden():
    with open(os.path.join(GOLDEN, "commit_rule_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        conf = np.array(c["conf"], dtype=np.float64)
        masked = np.array(c["masked"], dtype=bool)
        U = commit_rule(conf, masked, c["gamma"], c.get("rule", 0), c.get("min_adopt", 1))
        assert U.tolist() == c["adopt"], c


def test_commit_rule_min_adopt_one_is_the_fallback_rule():
    """Forced adoption of the top 1 together with the threshold is the threshold rule with
    its single-most-confident fallback, on random states (brute force)."""
    rng = np.random.default_rng(3)
    for _ in range(500):
        B = int(rng.integers(1, 9))
        conf = rng.choice([0.2, 0.5, 0.8, 0.9], size=B).astype(np.float64)
        masked = rng.random(B) < 0.7
        gamma = float(rng.choice([0.0, 0.5, 0.8, 0.95, 1.5]))
        c32 = conf.astype(np.float32)
        want = masked & (c32 >= np.float32(gamma))
        if masked.any() and not want.any():
            best = max((p for p in range(B) if masked[p]), key=lambda p: (c32[p], -p))
            want[best] = True
        assert commit_rule(conf, masked, gamma, 0, 1).tolist() == want.tolist()


def test_commit_rule_rejects_unknown_rules():
    with pytest.raises(ValueError):
        commit_rule(np.ones(2), np.ones(2, bool), 0.5, 7, 1)
    with pytest.raises(ValueError):
        commit_rule(np.ones(2), np.ones(2, bool), 0.5, 0, 0)
