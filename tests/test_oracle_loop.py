"""Pins of the oracle's whole step and block loop.

Closed forms of the loop (gamma <= 0, gamma > 1, zero LM head), invariants (monotone
commits, at most B steps, bidirectional symmetry, position equivariance), special
cases of the tower that reduce to torch library routines, and planted mistakes in
the oracle that those pins must catch.
"""
import copy

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.denoise as od
from oracle import OracleTower, oracle_generate, oracle_step, vocab_reduce
from tests.helpers import inputs, make_oracle, mini_workload


@pytest.fixture(scope="module")
def mini():
    w = mini_workload()
    orc, W = make_oracle(w)
    plens, tau, kv = inputs(w)
    return w, orc, W, plens, tau, kv


def _tower(w, W, mode="plain"):
    return OracleTower(W, H=w.H, Hkv=w.Hkv, hd=w.hd, eps=w.rms_eps, mode=mode)


# --------------------------------------------------------------------------- loop closed forms

def test_gamma_zero_commits_everything_in_one_step(mini):
    w, orc, W, plens, tau, kv = mini
    tok, cstep, steps, trace = oracle_generate(orc, w.n, w.B, tau, 0.0, kv)
    assert len(trace) == 1 and (steps == 1).all() and (cstep == 0).all()
    # tokens equal the argmax of one forward from the all-[MASK] block
    hf = orc.hidden(np.full((w.n, w.B), w.V), kv, range(w.n))
    z = orc.logits(hf.reshape(w.n * w.B, -1))
    _, arg, _ = vocab_reduce(z, tau.reshape(-1))
    assert np.array_equal(tok.reshape(-1), arg)


def test_gamma_above_one_takes_exactly_B_steps(mini):
    w, orc, W, plens, tau, kv = mini
    tok, cstep, steps, trace = oracle_generate(orc, w.n, w.B, tau, 1.5, kv)
    assert len(trace) == w.B and (steps == w.B).all()
    for r in trace:
        assert (r.U.sum(axis=1) == 1).all()
    for s in range(w.n):
        assert sorted(cstep[s].tolist()) == list(range(w.B))
        # each adopted position was the most confident masked one at its step
        for t, r in enumerate(trace):
            p = int(np.nonzero(r.U[s])[0][0])
            conf = np.where(np.isnan(r.conf[s]), -1, r.conf[s]).astype(np.float32)   # decided in fp32
            assert conf[p] == conf.max() and p == int(np.argmax(conf))


@pytest.mark.parametrize("k", [2, 3, 16])
def test_forced_top_k_above_gamma_one_adopts_k_per_step(mini, k):
    """gamma > 1 with the top k forced: exactly min(k, masked) positions per step, the k
    most confident in fp32 (lowest position on ties), ceil(B / k) steps."""
    w, orc, W, plens, tau, kv = mini
    tok, cstep, steps, trace = oracle_generate(orc, w.n, w.B, tau, 1.5, kv, min_adopt=k)
    assert (steps == -(-w.B // k)).all() and len(trace) == -(-w.B // k)
    for r in trace:
        for s in range(w.n):
            masked = ~np.isnan(r.conf[s])
            assert r.U[s].sum() == min(k, masked.sum())
            c32 = np.where(masked, r.conf[s], -1).astype(np.float32)
            order = sorted(np.nonzero(masked)[0].tolist(), key=lambda p: (-float(c32[p]), p))
            assert sorted(np.nonzero(r.U[s])[0].tolist()) == sorted(order[:k])


def test_left_to_right_commits_position_p_at_step_p(mini):
    """The mock-AR rule: one position per step, in position order, B steps; each adopted
    token is the argmax of that step's forward at that position."""
    w, orc, W, plens, tau, kv = mini
    tok, cstep, steps, trace = oracle_generate(orc, w.n, w.B, tau, 0.8, kv, rule=od.RULE_LEFT_TO_RIGHT)
    assert (steps == w.B).all() and len(trace) == w.B
    assert (cstep == np.arange(w.B)[None, :]).all()
    for t, r in enumerate(trace):
        assert (r.U.sum(axis=1) == 1).all() and r.U[:, t].all()
        assert np.array_equal(tok[:, t], r.arg[:, t])


def test_forced_top_k_with_threshold_is_a_superset_of_the_threshold_rule(mini):
    """From the same state, top-k forcing adopts everything the plain rule adopts, and more
    only where the plain rule adopted fewer than k."""
    w, orc, W, plens, tau, kv = mini
    tok = np.full((w.n, w.B), w.V)
    c = np.zeros((w.n, w.B), bool)
    r1 = oracle_step(orc, tok, c, tau, 0.8, kv)
    r3 = oracle_step(orc, tok, c, tau, 0.8, kv, min_adopt=3)
    assert (r3.U | ~r1.U).all()
    for s in range(w.n):
        assert r3.U[s].sum() == max(r1.U[s].sum(), 3)


@pytest.mark.parametrize("gamma", [0.3, 0.8, 0.95])
def test_loop_invariants(mini, gamma):
    w, orc, W, plens, tau, kv = mini
    tok, cstep, steps, trace = oracle_generate(orc, w.n, w.B, tau, gamma, kv)
    assert len(trace) <= w.B and (steps <= w.B).all() and (steps >= 1).all()
    assert (tok < w.V).all() and (cstep >= 0).all()
    prev_tok = np.full((w.n, w.B), w.V)
    prev_c = np.zeros((w.n, w.B), bool)
    for t, r in enumerate(trace):
        active = ~prev_c.all(axis=1)
        assert (r.U.sum(axis=1)[active] >= 1).all()
        assert not (r.U & prev_c).any()                       # committed positions are not re-adopted
        assert np.array_equal(r.tok[prev_c], prev_tok[prev_c])  # committed tokens never change
        assert np.array_equal(r.tok == w.V, ~r.committed)
        # every adopted position either clears gamma or is the single fallback
        for s in np.nonzero(active)[0]:
            c32 = r.conf[s].astype(np.float32)
            clear = (~prev_c[s]) & (c32 >= np.float32(gamma))
            if clear.any():
                assert np.array_equal(r.U[s], clear)
            else:
                assert r.U[s].sum() == 1
        prev_tok, prev_c = r.tok, r.committed
    assert prev_c.all()


def test_zero_lm_head_commits_in_position_order(mini):
    w, _, W, plens, tau, kv = mini
    W0 = dict(W)
    W0["lm_head"] = np.zeros_like(W["lm_head"])
    orc = _tower(w, W0)
    tok, cstep, steps, trace = oracle_generate(orc, w.n, w.B, tau, 0.8, kv)
    assert (tok == 0).all()
    for s in range(w.n):
        assert cstep[s].tolist() == list(range(w.B))
    np.testing.assert_allclose(trace[0].conf[~np.isnan(trace[0].conf)], 1.0 / w.V, rtol=1e-14)


# --------------------------------------------------------------------------- invariants of the tower

def _symmetric_weights(W):
    Ws = dict(W)
    Ws["pos_emb"] = np.zeros_like(W["pos_emb"])
    return Ws


def test_bidirectional_symmetry_of_masked_positions(mini):
    """With Pos = 0 every [MASK] position sees the same inputs and keys, so with no
    causal mask inside the block all masked positions get identical logits."""
    w, _, W, plens, tau, kv = mini
    orc = _tower(w, _symmetric_weights(W))
    tok = np.full((w.n, w.B), w.V)
    tok[:, 2] = 5
    hf = orc.hidden(tok, kv, range(w.n))
    for s in range(w.n):
        rows = [p for p in range(w.B) if p != 2]
        np.testing.assert_allclose(hf[s, rows], np.broadcast_to(hf[s, rows[0]], hf[s, rows].shape), rtol=1e-12)


def test_planted_causal_mask_breaks_symmetry(mini, monkeypatch):
    w, _, W, plens, tau, kv = mini

    def causal(q, k_pre, v_pre, k_blk, v_blk):
        out = np.empty_like(q)
        for p in range(q.shape[0]):   # position p sees the prefix and block keys 0..p only
            out[p:p + 1] = od.__dict__["_true_joint"](q[p:p + 1], k_pre, v_pre, k_blk[:p + 1], v_blk[:p + 1])
        return out

    monkeypatch.setitem(od.__dict__, "_true_joint", od.joint_attention)
    monkeypatch.setattr(od, "joint_attention", causal)
    orc = _tower(w, _symmetric_weights(W))
    hf = orc.hidden(np.full((w.n, w.B), w.V), kv, range(w.n))
    assert np.abs(hf[0, 1] - hf[0, 0]).max() > 1e-6


def test_position_equivariance(mini):
    """Permuting block positions together with their Pos rows permutes the outputs."""
    w, _, W, plens, tau, kv = mini
    orc = _tower(w, W)
    rng = np.random.default_rng(11)
    perm = rng.permutation(w.B)
    tok = np.full((w.n, w.B), w.V)
    tok[:, [1, 4]] = [[7, 3], [0, 9]]
    Wp = dict(W)
    Wp["pos_emb"] = W["pos_emb"][perm]
    hf = orc.hidden(tok, kv, range(w.n))
    hfp = _tower(w, Wp).hidden(tok[:, perm], kv, range(w.n))
    np.testing.assert_allclose(hfp, hf[:, perm], rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------- special cases vs torch

def _t(a):
    return torch.from_numpy(np.asarray(a, np.float64))


def _zero_layers(W, attn=True, mlp=True):
    W2 = copy.copy(W)
    for name in (["wq", "wk", "wv", "wo"] if attn else []) + (["w1", "w2"] if mlp else []):
        W2[name] = [np.zeros_like(a) for a in W[name]]
    return W2


def _embed(W, tok):
    return _t(W["tok_emb"])[torch.from_numpy(tok)] + _t(W["pos_emb"])[: tok.shape[1]]


def _pin_error_no_layers(orc, w, W, kv):
    tok = np.full((w.n, w.B), w.V)
    tok[:, 0] = 3
    x = _embed(W, tok)
    ref = F.linear(F.rms_norm(x, (w.d,), weight=_t(W["final_norm"]), eps=w.rms_eps), _t(W["lm_head"]))
    z = orc.logits(orc.hidden(tok, kv, range(w.n)).reshape(w.n * w.B, -1))
    return np.abs(z - ref.reshape(w.n * w.B, -1).numpy()).max() / np.abs(ref.numpy()).max()


def _pin_error_mlp_only(orc, w, W, kv):
    tok = np.full((w.n, w.B), w.V)
    tok[:, 1] = 4
    x = _embed(W, tok)
    for l in range(w.L):
        h = F.rms_norm(x, (w.d,), weight=_t(W["mlp_norm"][l]), eps=w.rms_eps)
        x = x + F.linear(F.gelu(F.linear(h, _t(W["w1"][l])), approximate="none"), _t(W["w2"][l]))
    ref = F.rms_norm(x, (w.d,), weight=_t(W["final_norm"]), eps=w.rms_eps).numpy()
    hf = orc.hidden(tok, kv, range(w.n))
    return np.abs(hf - ref).max() / np.abs(ref).max()


def _pin_error_attention_only(orc, w, W, kv):
    tok = np.full((w.n, w.B), w.V)
    tok[:, 5] = 8
    x = _embed(W, tok)
    for l in range(w.L):
        h = F.rms_norm(x, (w.d,), weight=_t(W["attn_norm"][l]), eps=w.rms_eps)
        outs = []
        for s in range(w.n):
            q = F.linear(h[s], _t(W["wq"][l])).reshape(w.B, w.H, w.hd).permute(1, 0, 2)
            k = F.linear(h[s], _t(W["wk"][l])).reshape(w.B, w.Hkv, w.hd)
            v = F.linear(h[s], _t(W["wv"][l])).reshape(w.B, w.Hkv, w.hd)
            kp, vp = kv(l, s)
            K = torch.cat([_t(kp), k]).permute(1, 0, 2)
            Vv = torch.cat([_t(vp), v]).permute(1, 0, 2)
            o = F.scaled_dot_product_attention(q[None], K[None], Vv[None], enable_gqa=True)[0]
            outs.append(o.permute(1, 0, 2).reshape(w.B, w.H * w.hd))
        x = x + F.linear(torch.stack(outs), _t(W["wo"][l]))
    ref = F.rms_norm(x, (w.d,), weight=_t(W["final_norm"]), eps=w.rms_eps).numpy()
    hf = orc.hidden(tok, kv, range(w.n))
    return np.abs(hf - ref).max() / np.abs(ref).max()


PINS = {
    "no_layers": (lambda W: _zero_layers(W), _pin_error_no_layers),
    "mlp_only": (lambda W: _zero_layers(W, attn=True, mlp=False), _pin_error_mlp_only),
    "attention_only": (lambda W: _zero_layers(W, attn=False, mlp=True), _pin_error_attention_only),
}


@pytest.mark.parametrize("pin", sorted(PINS))
def test_tower_special_cases_match_torch(mini, pin):
    w, _, W, plens, tau, kv = mini
    make_w, err = PINS[pin]
    Wz = make_w(W)
    assert err(_tower(w, Wz), w, Wz, kv) < 1e-12


def _gelu_tanh(x):
    return 0.5 * x * (1 + np.tanh(np.sqrt(2 / np.pi) * (x + 0.044715 * x ** 3)))


class _NoResidualTower(OracleTower):
    """Planted mistake: the MLP branch replaces the residual stream instead of adding to it."""

    def hidden(self, tok, kv, seqs, capture=None):
        return _drop_residual(self, self.W, tok, kv, seqs)


def _drop_residual(orc, W, tok, kv, seqs):
    S, B = tok.shape
    x = np.asarray(W["tok_emb"][tok.reshape(-1)], np.float64).reshape(S, B, orc.d) + orc._w("pos_emb")[None, :B]
    for l in range(orc.L):
        h2 = od.rmsnorm(x, orc._w("mlp_norm", l), orc.eps)
        x = od.gelu(h2 @ orc._w("w1", l).T) @ orc._w("w2", l).T
    return od.rmsnorm(x, orc._w("final_norm"), orc.eps)


@pytest.mark.parametrize("mistake", ["gelu_tanh", "no_residual", "transposed_gqa", "no_pos", "no_scale"])
def test_planted_mistakes_fail_a_pin(mini, monkeypatch, mistake):
    w, _, W, plens, tau, kv = mini
    if mistake == "gelu_tanh":
        monkeypatch.setattr(od, "gelu", _gelu_tanh)
        Wz = PINS["mlp_only"][0](W)
        assert _pin_error_mlp_only(_tower(w, Wz), w, Wz, kv) > 1e-6
    elif mistake == "no_residual":
        Wz = PINS["mlp_only"][0](W)
        orc = _NoResidualTower(Wz, H=w.H, Hkv=w.Hkv, hd=w.hd, eps=w.rms_eps)
        assert _pin_error_mlp_only(orc, w, Wz, kv) > 1e-6
    elif mistake in ("transposed_gqa", "no_scale"):
        true = od.joint_attention

        def wrong(q, kp, vp, kb, vb):
            if mistake == "transposed_gqa":   # head j -> K/V head j % Hkv instead of j // G
                Hkv = kb.shape[1]
                G = q.shape[1] // Hkv
                order = [(j % Hkv) * G + j // Hkv for j in range(q.shape[1])]
                return true(q[:, order], kp, vp, kb, vb)[:, np.argsort(order)]
            return true(q * np.sqrt(q.shape[2]), kp, vp, kb, vb)   # drops the 1/sqrt(hd) scale

        monkeypatch.setattr(od, "joint_attention", wrong)
        Wz = PINS["attention_only"][0](W)
        assert _pin_error_attention_only(_tower(w, Wz), w, Wz, kv) > 1e-6
    elif mistake == "no_pos":
        class NoPos(OracleTower):
            def _w(self, name, layer=-1):
                a = super()._w(name, layer)
                return np.zeros_like(a) if name == "pos_emb" else a
        Wz = PINS["no_layers"][0](W)
        orc = NoPos(Wz, H=w.H, Hkv=w.Hkv, hd=w.hd, eps=w.rms_eps)
        assert _pin_error_no_layers(orc, w, Wz, kv) > 1e-6


# --------------------------------------------------------------------------- bf16-faithful mode

def test_bf16_mode_rounds_only_at_storage_points(mini):
    w, _, W, plens, tau, kv = mini
    plain = _tower(w, W, "plain")
    faithful = _tower(w, W, "bf16")
    tok = np.full((w.n, w.B), w.V)
    hf_p = plain.hidden(tok, kv, range(w.n))
    hf_b = faithful.hidden(tok, kv, range(w.n))
    assert np.array_equal(od.round_bf16(hf_b), hf_b)          # hf is stored as bf16
    rel = np.abs(hf_b - hf_p).max() / np.abs(hf_p).max()
    assert 1e-5 < rel < 5e-2
    # logits stay unrounded
    z = faithful.logits(hf_b.reshape(w.n * w.B, -1))
    assert not np.array_equal(od.round_bf16(z), z)


def test_step_state_contract(mini):
    w, orc, W, plens, tau, kv = mini
    tok = np.full((w.n, w.B), w.V)
    bad = np.zeros((w.n, w.B), bool)
    bad[0, 0] = True          # committed but still [MASK]: not a valid state
    with pytest.raises(AssertionError):
        oracle_step(orc, tok, bad, tau, 0.8, kv)
