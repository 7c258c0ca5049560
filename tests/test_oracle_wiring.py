"""Pins of the oracle parts that the special cases of test_oracle_loop leave open.

* The per-sequence step count of the block loop, against two counts that do not use the
  loop's own counter: one plus the last step at which the sequence adopted a position,
  and the number of steps whose state still held a [MASK] in that sequence.
* The layer wiring with the attention and MLP branches both live.  With a block of one
  position and no prefix, each query row attends to exactly one key, its own, so the
  attention output of head j is the value row of K/V head j // (H / Hkv), whatever the
  queries are.  The whole tower then reduces to a chain of RMSNorm, matrix products and
  GELU that torch composes here on its own.
* The bf16 storage mode, against the same kind of chain with one prefix key (two keys
  per query, so the queries matter) and torch's round-to-nearest-even conversion at the
  storage points the mode declares.

Each pin is shown to fail on a planted mistake: the oracle's source is edited in memory
(one statement replaced) and run in its own module namespace.
"""
import inspect
import sys
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.denoise as od
from oracle import OracleTower, oracle_generate
from tests.helpers import inputs, make_oracle, mini_workload


def _mutant(func_name: str, old: str, new: str):
    """The oracle module with one statement of `func_name` (a function or a class) replaced."""
    src = inspect.getsource(od)
    body = inspect.getsource(getattr(od, func_name))
    assert src.count(body) == 1 and body.count(old) == 1, (func_name, old)
    mod = types.ModuleType("oracle_mutant")
    sys.modules["oracle_mutant"] = mod   # dataclasses look their module up while the class is built
    try:
        exec(compile(src.replace(body, body.replace(old, new)), "oracle_mutant", "exec"), mod.__dict__)
    finally:
        del sys.modules["oracle_mutant"]
    return mod


# --------------------------------------------------------------------------- per-sequence step counts

@pytest.fixture(scope="module")
def staggered():
    """A batch of four sequences whose loops end at different steps."""
    w = mini_workload(n=4, plen=("uniform", 0, 20))
    orc, W = make_oracle(w)
    plens, tau, kv = inputs(w)
    return w, orc, W, tau, kv


def _steps_pin_errors(steps, cstep, trace):
    """Differences between the loop's step counts and the two independent counts."""
    errs = []
    for s in range(steps.shape[0]):
        last = 1 + int(cstep[s].max())
        held_mask = sum(1 for r in trace if (~np.isnan(r.conf[s])).any())   # masked on entry to that step
        if steps[s] != last or steps[s] != held_mask:
            errs.append((s, int(steps[s]), last, held_mask))
    return errs


def test_step_counts_match_independent_counts(staggered):
    w, orc, W, tau, kv = staggered
    tok, cstep, steps, trace = oracle_generate(orc, w.n, w.B, tau, 0.8, kv)
    assert len(set(steps.tolist())) > 1, f"sequences must finish at different steps: {steps}"
    assert len(trace) == steps.max()
    assert _steps_pin_errors(steps, cstep, trace) == []


def test_step_count_pin_fails_on_counting_every_batch_step(staggered):
    w, orc, W, tau, kv = staggered
    bad = _mutant("oracle_generate", "steps += active", "steps += 1")
    tok, cstep, steps, trace = bad.oracle_generate(orc, w.n, w.B, tau, 0.8, kv)
    assert _steps_pin_errors(steps, cstep, trace) != []


def test_step_count_pin_fails_on_counting_from_the_new_state(staggered):
    w, orc, W, tau, kv = staggered
    # counting the sequences still masked AFTER the step drops each sequence's last step
    bad = _mutant("oracle_generate", "steps += active", "steps += ~r.committed.all(axis=1)")
    tok, cstep, steps, trace = bad.oracle_generate(orc, w.n, w.B, tau, 0.8, kv)
    assert _steps_pin_errors(steps, cstep, trace) != []


# --------------------------------------------------------------------------- two live branches

def _t(a):
    return torch.from_numpy(np.asarray(a, np.float64))


def _one_position(w):
    """A block of one position and no prefix on the mini tower shapes (GQA: 4 heads over 2)."""
    return w.with_(n=3, B=1, plen=("fixed", 0))


def _no_prefix(w):
    def kv(layer, seq):
        z = np.zeros((0, w.Hkv, w.hd))
        return z, z
    return kv


def _chain_one_key(w, W, tok, rnd=lambda t: t):
    """hf of blocks of one position with no prefix, composed with torch: per layer
    x += (v of head j // G for every head j) Wo^T, then x += gelu(rmsnorm(x) W1^T) W2^T.
    `rnd` is applied at the storage points (identity: plain float64)."""
    G = w.H // w.Hkv
    x = _t(W["tok_emb"])[torch.from_numpy(tok[:, 0])] + _t(W["pos_emb"])[0]
    for l in range(w.L):
        h = rnd(F.rms_norm(x, (w.d,), weight=_t(W["attn_norm"][l]), eps=w.rms_eps))
        v = rnd(F.linear(h, _t(W["wv"][l]))).reshape(-1, w.Hkv, w.hd)
        o = rnd(v[:, [j // G for j in range(w.H)], :].reshape(-1, w.H * w.hd))
        x = x + F.linear(o, _t(W["wo"][l]))
        h2 = rnd(F.rms_norm(x, (w.d,), weight=_t(W["mlp_norm"][l]), eps=w.rms_eps))
        x = x + F.linear(rnd(F.gelu(F.linear(h2, _t(W["w1"][l])), approximate="none")), _t(W["w2"][l]))
    return rnd(F.rms_norm(x, (w.d,), weight=_t(W["final_norm"]), eps=w.rms_eps)).numpy()


@pytest.fixture(scope="module")
def one_pos():
    w = _one_position(mini_workload())
    orc, W = make_oracle(w)
    tok = np.array([[w.V], [3], [17]])
    return w, W, tok


def _wiring_error(tower_cls, w, W, tok):
    orc = tower_cls(W, H=w.H, Hkv=w.Hkv, hd=w.hd, eps=w.rms_eps)
    hf = orc.hidden(tok, _no_prefix(w), range(tok.shape[0]))[:, 0]
    ref = _chain_one_key(w, W, tok)
    return np.abs(hf - ref).max() / np.abs(ref).max()


def test_two_branch_layer_matches_the_one_key_chain(one_pos):
    w, W, tok = one_pos
    assert w.H != w.Hkv   # the head mapping is part of the pin
    assert _wiring_error(OracleTower, w, W, tok) < 1e-12


@pytest.mark.parametrize("old,new", [
    # the MLP normalises the residual stream from before the attention update
    ("h2 = self._rnd(rmsnorm(x, self._w(\"mlp_norm\", l), self.eps))",
     "h2 = self._rnd(rmsnorm(x - o @ self._w(\"wo\", l).T, self._w(\"mlp_norm\", l), self.eps))"),
    # the attention output skips the output projection's residual (replaces x)
    ("x = x + o @ self._w(\"wo\", l).T", "x = o @ self._w(\"wo\", l).T"),
    # the MLP norm takes the attention norm's gain
    ("self._w(\"mlp_norm\", l)", "self._w(\"attn_norm\", l) * 1.5"),
])
def test_wiring_pin_fails_on_a_planted_mistake(one_pos, old, new):
    w, W, tok = one_pos
    bad = _mutant("OracleTower", old, new)
    assert _wiring_error(bad.OracleTower, w, W, tok) > 1e-6


def test_wiring_pin_fails_when_the_branches_swap_order(one_pos):
    """MLP first, then attention: computed by hand, it differs from the oracle."""
    w, W, tok = one_pos
    G = w.H // w.Hkv
    x = _t(W["tok_emb"])[torch.from_numpy(tok[:, 0])] + _t(W["pos_emb"])[0]
    for l in range(w.L):
        h2 = F.rms_norm(x, (w.d,), weight=_t(W["mlp_norm"][l]), eps=w.rms_eps)
        x = x + F.linear(F.gelu(F.linear(h2, _t(W["w1"][l])), approximate="none"), _t(W["w2"][l]))
        h = F.rms_norm(x, (w.d,), weight=_t(W["attn_norm"][l]), eps=w.rms_eps)
        v = F.linear(h, _t(W["wv"][l])).reshape(-1, w.Hkv, w.hd)
        x = x + F.linear(v[:, [j // G for j in range(w.H)], :].reshape(-1, w.H * w.hd), _t(W["wo"][l]))
    swapped = F.rms_norm(x, (w.d,), weight=_t(W["final_norm"]), eps=w.rms_eps).numpy()
    orc = OracleTower(W, H=w.H, Hkv=w.Hkv, hd=w.hd, eps=w.rms_eps)
    hf = orc.hidden(tok, _no_prefix(w), range(tok.shape[0]))[:, 0]
    assert np.abs(hf - swapped).max() / np.abs(swapped).max() > 1e-6


# --------------------------------------------------------------------------- bf16 storage mode

def _rnd_torch(t):
    return t.to(torch.bfloat16).to(torch.float64)


def _chain_two_keys(w, W, tok, kp, vp, rnd):
    """hf of one-position blocks with ONE prefix key per layer (kp[l], vp[l]: [S][Hkv][hd]),
    composed with torch: each query row softmaxes over two keys, the prefix key and its
    own, p = 1 / (1 + exp(s_own - s_pre)) on the prefix value."""
    G = w.H // w.Hkv
    heads = [j // G for j in range(w.H)]
    x = _t(W["tok_emb"])[torch.from_numpy(tok[:, 0])] + _t(W["pos_emb"])[0]
    for l in range(w.L):
        h = rnd(F.rms_norm(x, (w.d,), weight=_t(W["attn_norm"][l]), eps=w.rms_eps))
        q = rnd(F.linear(h, _t(W["wq"][l]))).reshape(-1, w.H, w.hd)
        k = rnd(F.linear(h, _t(W["wk"][l]))).reshape(-1, w.Hkv, w.hd)[:, heads]
        v = rnd(F.linear(h, _t(W["wv"][l]))).reshape(-1, w.Hkv, w.hd)[:, heads]
        kpre, vpre = _t(kp[l])[:, heads], _t(vp[l])[:, heads]
        s_pre = (q * kpre).sum(-1) / w.hd ** 0.5
        s_own = (q * k).sum(-1) / w.hd ** 0.5
        p_pre = 1.0 / (1.0 + torch.exp(s_own - s_pre))
        o = rnd((p_pre[..., None] * vpre + (1.0 - p_pre)[..., None] * v).reshape(-1, w.H * w.hd))
        x = x + F.linear(o, _t(W["wo"][l]))
        h2 = rnd(F.rms_norm(x, (w.d,), weight=_t(W["mlp_norm"][l]), eps=w.rms_eps))
        x = x + F.linear(rnd(F.gelu(F.linear(h2, _t(W["w1"][l])), approximate="none")), _t(W["w2"][l]))
    return rnd(F.rms_norm(x, (w.d,), weight=_t(W["final_norm"]), eps=w.rms_eps)).numpy()


@pytest.fixture(scope="module")
def one_key():
    w = _one_position(mini_workload())
    orc, W = make_oracle(w)
    rng = np.random.default_rng(5)
    S = 3
    # prefix keys/values exactly representable in bf16, as the stored caches are
    kp = [od.round_bf16(rng.standard_normal((S, w.Hkv, w.hd))) for _ in range(w.L)]
    vp = [od.round_bf16(rng.standard_normal((S, w.Hkv, w.hd))) for _ in range(w.L)]

    def kv(layer, seq):
        return kp[layer][seq:seq + 1], vp[layer][seq:seq + 1]

    tok = np.array([[w.V], [3], [17]])
    return w, W, tok, kp, vp, kv


def _bf16_error(tower_cls, w, W, tok, kp, vp, kv, mode="bf16"):
    orc = tower_cls(W, H=w.H, Hkv=w.Hkv, hd=w.hd, eps=w.rms_eps, mode=mode)
    hf = orc.hidden(tok, kv, range(tok.shape[0]))[:, 0]
    ref = _chain_two_keys(w, W, tok, kp, vp, _rnd_torch)
    return np.abs(hf - ref).max() / np.abs(ref).max()


def test_bf16_mode_matches_the_hand_rounded_chain(one_key):
    w, W, tok, kp, vp, kv = one_key
    assert _bf16_error(OracleTower, w, W, tok, kp, vp, kv) < 1e-12
    # the same chain without rounding is the plain mode, and the two differ
    plain = _chain_two_keys(w, W, tok, kp, vp, lambda t: t)
    orc = OracleTower(W, H=w.H, Hkv=w.Hkv, hd=w.hd, eps=w.rms_eps, mode="plain")
    hf = orc.hidden(tok, kv, range(tok.shape[0]))[:, 0]
    assert np.abs(hf - plain).max() / np.abs(plain).max() < 1e-12
    assert np.abs(plain - _chain_two_keys(w, W, tok, kp, vp, _rnd_torch)).max() > 1e-4


@pytest.mark.parametrize("old,new", [
    # q kept unrounded
    ("q = self._rnd(h @ self._w(\"wq\", l).T)", "q = (h @ self._w(\"wq\", l).T)"),
    # the attention output kept unrounded
    ("o = self._rnd(o.reshape(S, B, H * hd))", "o = o.reshape(S, B, H * hd)"),
    # the MLP activation kept unrounded
    ("u = self._rnd(gelu(h2 @ self._w(\"w1\", l).T))", "u = gelu(h2 @ self._w(\"w1\", l).T)"),
    # the final normed state kept unrounded
    ("return self._rnd(rmsnorm(x, self._w(\"final_norm\"), self.eps))",
     "return rmsnorm(x, self._w(\"final_norm\"), self.eps)"),
])
def test_bf16_pin_fails_on_a_missing_rounding(one_key, old, new):
    w, W, tok, kp, vp, kv = one_key
    bad = _mutant("OracleTower", old, new)
    assert _bf16_error(bad.OracleTower, w, W, tok, kp, vp, kv) > 1e-6


def test_bf16_pin_fails_on_truncation(one_key, monkeypatch):
    """Rounding toward zero instead of to nearest even."""
    w, W, tok, kp, vp, kv = one_key

    def trunc(x):
        x = np.asarray(x, dtype=np.float64)
        _, e = np.frexp(x)
        e = np.maximum(e, -125)
        return np.ldexp(np.trunc(np.ldexp(x, 8 - e)), e - 8)

    monkeypatch.setattr(od, "round_bf16", trunc)
    assert _bf16_error(OracleTower, w, W, tok, kp, vp, kv) > 1e-6
