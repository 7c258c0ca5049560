"""Plain float64 oracle of one block-diffusion denoising step and of the block loop.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's
CPU baseline; never by the product path.

What is computed, and where it comes from:

* Reverse process.  A network reads a block in which some positions hold the
  special [MASK] token and predicts a token for every masked position in parallel
  (PredNext, "人工知能は拡散言語モデルの夢を見るか？", section
  "拡散言語モデルのLLMへの応用").  The [MASK] id is V, an extra embedding row; the
  LM head has V outputs so it can never emit [MASK].
* Network.  The denoiser tower attends bidirectionally inside the block and
  cross-attends to the frozen, causal context tower through that tower's cached
  keys/values (poko-everyday.com Nemotron-TwoTower news item, section
  技術/ビジネス面).  Read here as ONE softmax per query over [prefix keys ; block
  keys] with no mask; layer l of the denoiser reads prefix K/V layer l; query head
  j uses K/V head floor(j / (H / Hkv)).  Pre-norm residual layers with RMSNorm
  (eps 1e-6), an ungated GELU MLP (erf form) of width F, a final RMSNorm, no biases.
  A learned per-block-position row Pos[p] is added to the token embedding; without
  it every masked position would see identical inputs and produce identical
  predictions.
* Confidence.  conf_p is the largest softmax probability of the logits of position
  p scaled by that position's inverse temperature tau_p; the prediction is the
  lowest vocabulary id among the maximal scaled logits.
* Commit rule and loop (PredNext, same article, section
  "拡散言語モデルで推論するには", steps 1-5; dzen.guru "NVIDIA Nemotron 70B
  генерирует текст…", section "Что нового": blocks of 16 refined over several
  iterations, threshold gamma trades quality for speed).  Start from an all-[MASK]
  block; run the network; adopt every masked position whose confidence is at
  least gamma; if none is, adopt the single most confident masked position
  (lowest position on ties); the rest stay [MASK]; repeat until no [MASK] is left.
  Adopted tokens never change.  Every step adopts at least one position, so a
  block of B ends in at most B steps.  Variants (commit_rule): the same step 3 names
  forcing the top few positions as another way (adopt the min_adopt most confident
  together with those clearing gamma; min_adopt = 1 is the rule above), and the
  pages' mock-AR mode (dzen, section "Что нового": one token per step through the
  diffusion tower) is read as left-to-right order.

* Mixture-of-experts MLP (optional; dzen, section "Что нового": the tower's layers
  are MoE layers in which 6 of 128 experts plus 2 shared ones are active per token).
  Readings: a router row per expert scores the normed MLP input; each token takes its
  top_k experts by score (lowest expert id on ties) with gates given by a softmax over
  the chosen scores; every expert, routed or shared, is the same ungated GELU MLP of
  width d_expert; shared experts always apply with weight 1; the MoE replaces the
  denoiser's dense MLP in every layer.  See moe_ffn.

Precision.  Everything is float64.  Mode "bf16" additionally rounds to the nearest
bfloat16 (ties to even) exactly at the points where the GPU stores bfloat16: the
normed GEMM inputs (h, h2, hf), q/k/v, the attention output o and the MLP
activation u.  Logits are never rounded.  Decisions that turn floats into
integers (argmax, conf >= gamma, the fallback choice, the experts a token is routed
to) are taken on float32 roundings of the float64 values, the precision the kernels
decide in.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np
from scipy.special import erf


# ----------------------------------------------------------------------------- elementwise


def round_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value of each float64 element, ties to even (finite inputs).

    bfloat16 keeps 8 significant bits and float32's exponent range.  For
    x = m * 2**e with 0.5 <= |m| < 1 the representable neighbours are multiples of
    2**(e-8); below 2**-126 the spacing stays 2**-133 (subnormals).
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    return np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x**2) + eps) * g over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU: 0.5 * x * (1 + erf(x / sqrt(2)))."""
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


# ----------------------------------------------------------------------------- mixture of experts


def moe_route(scores: np.ndarray, top_k: int):
    """Experts and gates of each row from router scores [R][E] (float64).

    The top_k experts of a row are those with the largest float32-rounded scores, the
    lowest expert id first among equal scores, listed by rank; the gates are a softmax
    over the chosen float64 scores (they sum to 1).  Returns (experts [R][top_k] int64,
    gates [R][top_k] float64).
    """
    R, E = scores.shape
    if not 1 <= top_k <= E:
        raise ValueError("top_k must be in [1, E]")
    s32 = scores.astype(np.float32)
    experts = np.empty((R, top_k), dtype=np.int64)
    gates = np.empty((R, top_k))
    for r in range(R):
        ranked = sorted(range(E), key=lambda e: (-float(s32[r, e]), e))[:top_k]
        experts[r] = ranked
        sel = scores[r, ranked]
        w = np.exp(sel - sel.max())
        gates[r] = w / w.sum()
    return experts, gates


def moe_ffn(h2: np.ndarray, router, w1, w2, sw1, sw2, top_k: int, rnd=lambda a: a):
    """Mixture-of-experts MLP output for normed inputs h2 [R][d] (float64).

    router [E][d]; w1[e] [d_expert][d] and w2[e] [d][d_expert] for the routed experts;
    sw1[s], sw2[s] likewise for the shared experts (empty sequences for none).  Expert
    weights are read one expert at a time (any indexable container).  With expert(h) =
    gelu(h W1^T) W2^T (its GELU output passed through rnd, the storage rounding):

        y_r = sum over the row's chosen experts e of gate_{r,e} * expert_e(h2_r)
              + sum over shared experts s of shared_s(h2_r)

    Returns (y [R][d], experts [R][top_k], gates [R][top_k], scores [R][E]).
    """
    scores = h2 @ np.asarray(router, np.float64).T
    experts, gates = moe_route(scores, top_k)
    y = np.zeros_like(h2)
    for e in np.unique(experts):
        rows, slot = np.nonzero(experts == e)
        u = rnd(gelu(h2[rows] @ np.asarray(w1[e], np.float64).T))
        y[rows] += gates[rows, slot][:, None] * (u @ np.asarray(w2[e], np.float64).T)
    for s in range(len(sw1)):
        u = rnd(gelu(h2 @ np.asarray(sw1[s], np.float64).T))
        y += u @ np.asarray(sw2[s], np.float64).T
    return y, experts, gates, scores


# ----------------------------------------------------------------------------- attention


def joint_attention(q: np.ndarray, k_pre: np.ndarray, v_pre: np.ndarray, k_blk: np.ndarray,
                    v_blk: np.ndarray, causal: bool = False) -> np.ndarray:
    """Block queries against [prefix keys ; block keys], one softmax per query row.

    q [B][H][hd]; k_pre, v_pre [P][Hkv][hd] (P may be 0); k_blk, v_blk [B][Hkv][hd].
    Returns o [B][H][hd].  Query head j reads K/V head j // (H // Hkv).  No mask for the
    denoiser; causal=True (the context tower) shows block query p the whole prefix and the
    block keys 0..p only.
    """
    Bq, H, hd = q.shape
    Hkv = k_blk.shape[1]
    P = k_pre.shape[0]
    G = H // Hkv
    o = np.empty((Bq, H, hd), dtype=np.float64)
    for j in range(H):
        g = j // G
        K = np.concatenate([k_pre[:, g, :], k_blk[:, g, :]], axis=0)
        Vv = np.concatenate([v_pre[:, g, :], v_blk[:, g, :]], axis=0)
        s = (q[:, j, :] @ K.T) / np.sqrt(hd)
        if causal:
            later = np.arange(k_blk.shape[0])[None, :] > np.arange(Bq)[:, None]
            s[:, P:][later] = -np.inf
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        o[:, j, :] = p @ Vv
    return o


# ----------------------------------------------------------------------------- tower

KVProvider = Callable[[int, int], Tuple[np.ndarray, np.ndarray]]   # (layer, seq) -> (K, V) [P][Hkv][hd]


class OracleTower:
    """The denoiser tower with its weights held as float64.

    `weights` maps names to arrays holding the stored values exactly (float32, or
    bfloat16 widened to float32): tok_emb [V+1][d], pos_emb [B][d], final_norm [d],
    lm_head [V][d], and per-layer lists wq [H*hd][d], wk/wv [Hkv*hd][d],
    wo [d][H*hd], w1 [F][d], w2 [d][F], attn_norm [d], mlp_norm [d].

    An optional "moe" entry replaces every layer's dense MLP with a mixture of experts
    (moe_ffn): a dict with top_k and per-layer lists router [E][d], w1 [E][d_expert][d],
    w2 [E][d][d_expert], sw1 [n_shared][d_expert][d], sw2 [n_shared][d][d_expert] (the
    per-layer entries index by expert; w1/w2 of the dense MLP are then unused).
    """

    def __init__(self, weights: Dict[str, object], *, H: int, Hkv: int, hd: int, eps: float = 1e-6,
                 mode: str = "plain"):
        if mode not in ("plain", "bf16"):
            raise ValueError(mode)
        self.W = weights
        self.H, self.Hkv, self.hd, self.eps, self.mode = H, Hkv, hd, eps, mode
        self.L = len(weights["wq"])
        self.moe = weights.get("moe")
        self.V = weights["lm_head"].shape[0]
        self.d = weights["lm_head"].shape[1]
        self._f64: Dict[Tuple[str, int], np.ndarray] = {}

    def _w(self, name: str, layer: int = -1) -> np.ndarray:
        key = (name, layer)
        if key not in self._f64:
            a = self.W[name] if layer < 0 else self.W[name][layer]
            self._f64[key] = np.asarray(a, dtype=np.float64)
        return self._f64[key]

    def _rnd(self, a: np.ndarray) -> np.ndarray:
        return round_bf16(a) if self.mode == "bf16" else a

    def hidden(self, tok: np.ndarray, kv: KVProvider, seqs: Sequence[int],
               capture: Optional[dict] = None) -> np.ndarray:
        """Final-normed hidden states hf [S][B][d] for token blocks tok [S][B].

        `seqs[s]` is the batch index of row-block s, passed to `kv` to fetch its prefix.
        """
        S, B = tok.shape
        H, Hkv, hd = self.H, self.Hkv, self.hd
        E = self.W["tok_emb"]
        x = np.asarray(E[tok.reshape(-1)], dtype=np.float64).reshape(S, B, self.d)
        x = x + self._w("pos_emb")[None, :B, :]
        for l in range(self.L):
            h = self._rnd(rmsnorm(x, self._w("attn_norm", l), self.eps))
            q = self._rnd(h @ self._w("wq", l).T).reshape(S, B, H, hd)
            k = self._rnd(h @ self._w("wk", l).T).reshape(S, B, Hkv, hd)
            v = self._rnd(h @ self._w("wv", l).T).reshape(S, B, Hkv, hd)
            o = np.empty((S, B, H, hd))
            for s in range(S):
                kp, vp = kv(l, seqs[s])
                o[s] = joint_attention(q[s], np.asarray(kp, np.float64), np.asarray(vp, np.float64),
                                       k[s], v[s])
            o = self._rnd(o.reshape(S, B, H * hd))
            x = x + o @ self._w("wo", l).T
            h2 = self._rnd(rmsnorm(x, self._w("mlp_norm", l), self.eps))
            if self.moe is not None:
                m = self.moe
                y, ex, gt, sc = moe_ffn(h2.reshape(S * B, self.d), m["router"][l], m["w1"][l], m["w2"][l],
                                        m["sw1"][l], m["sw2"][l], m["top_k"], self._rnd)
                x = x + y.reshape(S, B, self.d)
                if capture is not None:
                    capture.setdefault("experts", []).append(ex.reshape(S, B, -1))
                    capture.setdefault("gates", []).append(gt.reshape(S, B, -1))
                    capture.setdefault("scores", []).append(sc.reshape(S, B, -1))
            else:
                u = self._rnd(gelu(h2 @ self._w("w1", l).T))
                x = x + u @ self._w("w2", l).T
            if capture is not None:
                capture.setdefault("x", []).append(x.copy())
        return self._rnd(rmsnorm(x, self._w("final_norm"), self.eps))

    def logits(self, hf_rows: np.ndarray) -> np.ndarray:
        """z = hf Wlm^T for rows hf_rows [R][d] (float64, never rounded)."""
        return hf_rows @ self._w("lm_head").T


class OracleContextTower:
    """The frozen context tower over a committed block, float64.

    The pages describe it as the causal tower whose cached K/V the denoiser reads
    (poko, section 技術/ビジネス面; dzen, section Что нового: frozen).  Readings: the
    denoiser's shapes with weights of its own (tok_emb [V+1][d]; per layer wq, wk, wv,
    wo, w1, w2, attn_norm, mlp_norm), no position table (the causal mask orders its
    tokens), each block query attending causally inside the block and to the whole
    cached prefix.  block_kv returns, per layer, the k and v of the block's tokens: what
    is appended to the cache that layer l of the denoiser reads.
    """

    def __init__(self, weights: Dict[str, object], *, H: int, Hkv: int, hd: int, eps: float = 1e-6):
        self.W = weights
        self.H, self.Hkv, self.hd, self.eps = H, Hkv, hd, eps
        self.L = len(weights["wq"])
        self.d = weights["tok_emb"].shape[1]

    def _w(self, name: str, layer: int) -> np.ndarray:
        return np.asarray(self.W[name][layer], dtype=np.float64)

    def ar_step(self, tok: np.ndarray, kv: KVProvider, seqs: Sequence[int]):
        """One autoregressive decode step (dzen, section Что нового: the classic AR mode;
        read as the context tower used as an AR model with a final norm and LM head of
        its own, final_norm [d] and lm_head [V][d]): the full tower over one token per
        sequence, tok [S], attending to its cached prefix and itself.

        Returns ([(k [S][1][Hkv][hd], v ...) per layer], logits z [S][V] float64); the
        next token is the lowest id of the largest fp32 logit."""
        S = tok.shape[0]
        H, Hkv, hd = self.H, self.Hkv, self.hd
        x = np.asarray(self.W["tok_emb"][tok.reshape(-1)], dtype=np.float64).reshape(S, 1, self.d)
        out = []
        for l in range(self.L):
            h = rmsnorm(x, self._w("attn_norm", l), self.eps)
            q = (h @ self._w("wq", l).T).reshape(S, 1, H, hd)
            k = (h @ self._w("wk", l).T).reshape(S, 1, Hkv, hd)
            v = (h @ self._w("wv", l).T).reshape(S, 1, Hkv, hd)
            out.append((k, v))
            o = np.empty((S, 1, H, hd))
            for s in range(S):
                kp, vp = kv(l, seqs[s])
                o[s] = joint_attention(q[s], np.asarray(kp, np.float64), np.asarray(vp, np.float64), k[s], v[s],
                                       causal=True)
            x = x + o.reshape(S, 1, H * hd) @ self._w("wo", l).T
            h2 = rmsnorm(x, self._w("mlp_norm", l), self.eps)
            x = x + gelu(h2 @ self._w("w1", l).T) @ self._w("w2", l).T
        hf = rmsnorm(x.reshape(S, self.d), np.asarray(self.W["final_norm"], np.float64), self.eps)
        return out, hf @ np.asarray(self.W["lm_head"], np.float64).T

    def block_kv(self, tok: np.ndarray, kv: KVProvider, seqs: Sequence[int]):
        """[(k [S][B][Hkv][hd], v [S][B][Hkv][hd]) for each layer] of token blocks tok [S][B]."""
        S, B = tok.shape
        H, Hkv, hd = self.H, self.Hkv, self.hd
        x = np.asarray(self.W["tok_emb"][tok.reshape(-1)], dtype=np.float64).reshape(S, B, self.d)
        out = []
        for l in range(self.L):
            h = rmsnorm(x, self._w("attn_norm", l), self.eps)
            q = (h @ self._w("wq", l).T).reshape(S, B, H, hd)
            k = (h @ self._w("wk", l).T).reshape(S, B, Hkv, hd)
            v = (h @ self._w("wv", l).T).reshape(S, B, Hkv, hd)
            out.append((k, v))
            if l == self.L - 1:
                break          # nothing above the last layer's K/V is read
            o = np.empty((S, B, H, hd))
            for s in range(S):
                kp, vp = kv(l, seqs[s])
                o[s] = joint_attention(q[s], np.asarray(kp, np.float64), np.asarray(vp, np.float64), k[s], v[s],
                                       causal=True)
            x = x + o.reshape(S, B, H * hd) @ self._w("wo", l).T
            h2 = rmsnorm(x, self._w("mlp_norm", l), self.eps)
            x = x + gelu(h2 @ self._w("w1", l).T) @ self._w("w2", l).T
        return out


# ----------------------------------------------------------------------------- reduction + commit


def vocab_reduce(z: np.ndarray, tau: np.ndarray):
    """Per row: conf = max softmax prob of tau*z, arg = lowest id of the max, gap = p1 - p2.

    z [R][V] float64, tau [R].  arg is decided on the float32 rounding of tau*z.
    """
    s = np.asarray(tau, np.float64)[:, None] * z
    arg = np.argmax(s.astype(np.float32), axis=1)          # first maximum = lowest id
    m = s.max(axis=1, keepdims=True)
    Z = np.exp(s - m).sum(axis=1)
    conf = 1.0 / Z
    s2 = np.partition(s, s.shape[1] - 2, axis=1)[:, -2]
    p2 = np.exp(s2 - m[:, 0]) / Z
    return conf, arg.astype(np.int64), conf - p2


RULE_THRESHOLD, RULE_LEFT_TO_RIGHT = 0, 1


def commit_rule(conf: np.ndarray, masked: np.ndarray, gamma: float, rule: int = RULE_THRESHOLD,
                min_adopt: int = 1) -> np.ndarray:
    """Positions adopted this step.

    RULE_THRESHOLD (PredNext, section 拡散言語モデルで推論するには, step 3: adopt the
    positions whose output clears the threshold; the same step names forcing the top few
    as another way): masked positions with conf >= gamma, together with the min_adopt
    most confident masked positions (ties to the lowest position).  min_adopt = 1 is the
    fixed fallback: the single most confident position when none clears gamma.

    RULE_LEFT_TO_RIGHT (dzen, section Что нового: the mock-AR mode, one token per step
    through the diffusion tower, read as autoregressive order): the lowest masked
    position; gamma and min_adopt play no part.

    Decided in float32.  A block with no masked position adopts nothing.
    """
    masked = np.asarray(masked, bool)
    U = np.zeros_like(masked)
    if not masked.any():
        return U
    if rule == RULE_LEFT_TO_RIGHT:
        U[int(np.argmax(masked))] = True
        return U
    if rule != RULE_THRESHOLD or min_adopt < 1:
        raise ValueError("unknown commit rule")
    c32 = np.asarray(conf, np.float64).astype(np.float32)
    U = masked & (c32 >= np.float32(gamma))
    ranked = sorted(np.nonzero(masked)[0].tolist(), key=lambda p: (-float(c32[p]), p))
    U[ranked[:min_adopt]] = True
    return U


@dataclasses.dataclass
class StepResult:
    conf: np.ndarray        # [S][B] float64 (nan where committed on entry)
    arg: np.ndarray         # [S][B] int64 (-1 where committed on entry)
    gap: np.ndarray         # [S][B] p1 - p2 (nan where committed on entry)
    U: np.ndarray           # [S][B] bool, adopted this step
    tok: np.ndarray         # [S][B] tokens after the step
    committed: np.ndarray   # [S][B] bool after the step
    z: Optional[np.ndarray] = None   # [S][B][V] logits of masked rows (nan elsewhere) if kept
    zmax: Optional[np.ndarray] = None   # [S][B] max_v |z| of masked rows (nan elsewhere): the scale of a row's logits


def oracle_step(tower: OracleTower, tok: np.ndarray, committed: np.ndarray, tau: np.ndarray,
                gamma: float, kv: KVProvider, seqs: Optional[Sequence[int]] = None,
                keep_logits: bool = False, rule: int = RULE_THRESHOLD, min_adopt: int = 1) -> StepResult:
    """One denoising step for S independent sequences from state (tok, committed)."""
    S, B = tok.shape
    seqs = list(range(S)) if seqs is None else list(seqs)
    masked = ~committed.astype(bool)
    assert np.array_equal(tok == tower.V, masked), "state must hold [MASK] exactly at uncommitted positions"
    hf = tower.hidden(tok, kv, seqs)
    rows = np.nonzero(masked.reshape(-1))[0]
    conf = np.full(S * B, np.nan)
    arg = np.full(S * B, -1, dtype=np.int64)
    gap = np.full(S * B, np.nan)
    zmax = np.full(S * B, np.nan)
    z_all = None
    if rows.size:
        z = tower.logits(hf.reshape(S * B, -1)[rows])
        c, a, g = vocab_reduce(z, tau.reshape(-1)[rows])
        conf[rows], arg[rows], gap[rows] = c, a, g
        zmax[rows] = np.abs(z).max(axis=1)
        if keep_logits:
            z_all = np.full((S * B, tower.V), np.nan)
            z_all[rows] = z
            z_all = z_all.reshape(S, B, tower.V)
    conf, arg, gap = conf.reshape(S, B), arg.reshape(S, B), gap.reshape(S, B)
    U = np.zeros((S, B), dtype=bool)
    for s in range(S):
        U[s] = commit_rule(conf[s], masked[s], gamma, rule, min_adopt)
    new_tok = np.where(U, arg, tok)
    new_c = committed.astype(bool) | U
    return StepResult(conf, arg, gap, U, new_tok, new_c, z_all, zmax.reshape(S, B))


def oracle_generate_blocks(tower: OracleTower, context: OracleContextTower, n_blocks: int, S: int, B: int,
                           tau: np.ndarray, gamma: float, kv: KVProvider, seqs: Optional[Sequence[int]] = None,
                           cache_bf16: bool = True, rule: int = RULE_THRESHOLD, min_adopt: int = 1,
                           return_kv: bool = False):
    """Generation of n_blocks consecutive blocks: each block is refined to completion by
    the block loop; the context tower then runs over its tokens and their K/V (rounded
    to bf16 when the cache holds bf16) are appended to every layer's cache, so the next
    block sees them as prefix.  The same inverse temperatures serve every block.

    Returns (tok [n_blocks][S][B], commit_step [n_blocks][S][B], steps [n_blocks][S]) and,
    with return_kv, the appended {(layer, seq): [(k, v) [B][Hkv][hd] per block]} as stored.
    """
    seqs = list(range(S)) if seqs is None else list(seqs)
    added: Dict[Tuple[int, int], List[Tuple[np.ndarray, np.ndarray]]] = {}

    def kv_now(l: int, s: int):
        K, V = kv(l, s)
        extra = added.get((l, s), [])
        if not extra:
            return K, V
        return (np.concatenate([np.asarray(K, np.float64)] + [e[0] for e in extra], axis=0),
                np.concatenate([np.asarray(V, np.float64)] + [e[1] for e in extra], axis=0))

    toks, csteps, steps = [], [], []
    for _ in range(n_blocks):
        tok, cs, st, _ = oracle_generate(tower, S, B, tau, gamma, kv_now, seqs, keep_trace=False, rule=rule,
                                         min_adopt=min_adopt)
        toks.append(tok)
        csteps.append(cs)
        steps.append(st)
        kvs = context.block_kv(tok, kv_now, seqs)
        for l, (k, v) in enumerate(kvs):
            for i, s in enumerate(seqs):
                kk, vv = (round_bf16(k[i]), round_bf16(v[i])) if cache_bf16 else (k[i], v[i])
                added.setdefault((l, s), []).append((kk, vv))
    if return_kv:
        return np.stack(toks), np.stack(csteps), np.stack(steps), added
    return np.stack(toks), np.stack(csteps), np.stack(steps)


def oracle_ar_decode(context: OracleContextTower, first: np.ndarray, n_steps: int, kv: KVProvider,
                     seqs: Optional[Sequence[int]] = None, cache_bf16: bool = True):
    """Greedy AR decoding with the context tower: n_steps steps from tokens first [S];
    each step appends the input token's K/V (rounded to bf16 when the cache holds bf16)
    and predicts the next token (argmax of the fp32 logits, lowest id on ties).

    Returns tokens [S][n_steps] (the prediction of every step)."""
    S = first.shape[0]
    seqs = list(range(S)) if seqs is None else list(seqs)
    added: Dict[Tuple[int, int], List[Tuple[np.ndarray, np.ndarray]]] = {}

    def kv_now(l: int, s: int):
        K, V = kv(l, s)
        extra = added.get((l, s), [])
        if not extra:
            return K, V
        return (np.concatenate([np.asarray(K, np.float64)] + [e[0] for e in extra], axis=0),
                np.concatenate([np.asarray(V, np.float64)] + [e[1] for e in extra], axis=0))

    tok = np.asarray(first, np.int64)
    outs = []
    for _ in range(n_steps):
        kvs, z = context.ar_step(tok, kv_now, seqs)
        for l, (k, v) in enumerate(kvs):
            for i, s in enumerate(seqs):
                kk, vv = (round_bf16(k[i]), round_bf16(v[i])) if cache_bf16 else (k[i], v[i])
                added.setdefault((l, s), []).append((kk, vv))
        tok = np.argmax(z.astype(np.float32), axis=1).astype(np.int64)
        outs.append(tok)
    return np.stack(outs, axis=1)


def oracle_generate(tower: OracleTower, S: int, B: int, tau: np.ndarray, gamma: float, kv: KVProvider,
                    seqs: Optional[Sequence[int]] = None, keep_trace: bool = True, rule: int = RULE_THRESHOLD,
                    min_adopt: int = 1):
    """Run the block loop from an all-[MASK] block until every position is adopted.

    Returns (tok [S][B], commit_step [S][B], steps [S], trace: list of StepResult).
    steps[s] counts the steps in which sequence s still had a masked position.
    """
    tok = np.full((S, B), tower.V, dtype=np.int64)
    committed = np.zeros((S, B), dtype=bool)
    commit_step = np.full((S, B), -1, dtype=np.int64)
    steps = np.zeros(S, dtype=np.int64)
    trace: List[StepResult] = []
    t = 0
    while not committed.all():
        active = ~committed.all(axis=1)
        r = oracle_step(tower, tok, committed, tau, gamma, kv, seqs, rule=rule, min_adopt=min_adopt)
        assert (r.U.sum(axis=1)[active] >= 1).all(), "an active sequence must adopt at least one position"
        commit_step[r.U] = t
        steps += active
        tok, committed = r.tok, r.committed
        if keep_trace:
            trace.append(r)
        t += 1
        assert t <= B, "the loop must end within B steps"
    return tok, commit_step, steps, trace
