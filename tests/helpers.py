"""Shared test helpers: small towers, oracle construction from synthetic inputs."""
import numpy as np

from synth import Workload, draw_tower, draw_prefix_lengths, draw_inv_temp, draw_prefix_kv, f32_from_bf16_bits


def mini_workload(**kw) -> Workload:
    """A tiny tower for oracle loop tests: weights wide enough that confidences spread."""
    base = dict(name="mini", tower="mini", n=2, plen=("uniform", 0, 12), B=8, d=32, H=4, Hkv=2, hd=8, L=2,
                F=128, V=50, dtype="f32", weight_std=0.25)
    base.update(kw)
    return Workload(**base)


class _Widened:
    """Experts of one layer, widened to float32 one at a time when the oracle reads them."""

    def __init__(self, a, tw):
        self.a, self.tw = a, tw

    def __getitem__(self, e):
        return self.tw.as_f32(self.a[e])

    def __len__(self):
        return self.a.shape[0]


def oracle_weights(tw, moe=None) -> dict:
    """Stored tower values widened exactly to float32, keyed as the oracle expects;
    `moe` (synth.MoeInputs) adds the mixture of experts."""
    f = lambda a: None if a is None else tw.as_f32(a)  # noqa: E731  (the context tower has no pos/final/head)
    W = dict(tok_emb=f(tw.tok_emb), pos_emb=f(tw.pos_emb), final_norm=f(tw.final_norm), lm_head=f(tw.lm_head),
             wq=[f(a) for a in tw.wq], wk=[f(a) for a in tw.wk], wv=[f(a) for a in tw.wv],
             wo=[f(a) for a in tw.wo], w1=[f(a) for a in tw.w1], w2=[f(a) for a in tw.w2],
             attn_norm=[f(a) for a in tw.attn_norm], mlp_norm=[f(a) for a in tw.mlp_norm])
    if moe is not None:
        W["moe"] = dict(top_k=moe.w.moe[1], router=[f(a) for a in moe.router],
                        w1=[_Widened(a, tw) for a in moe.w1], w2=[_Widened(a, tw) for a in moe.w2],
                        sw1=[_Widened(a, tw) for a in moe.sw1], sw2=[_Widened(a, tw) for a in moe.sw2])
    return W


def kv_provider(w: Workload, plens):
    cache = {}

    def kv(layer, seq):
        key = (layer, seq)
        if key not in cache:
            k = draw_prefix_kv(w, layer, seq, int(plens[seq]), "k")
            v = draw_prefix_kv(w, layer, seq, int(plens[seq]), "v")
            if w.dtype == "bf16":
                k, v = f32_from_bf16_bits(k), f32_from_bf16_bits(v)
            cache[key] = (k, v)
        return cache[key]

    return kv


def make_oracle(w: Workload, mode: str = "plain", weights: dict = None):
    from oracle import OracleTower
    tw = draw_tower(w)
    W = weights if weights is not None else oracle_weights(tw)
    return OracleTower(W, H=w.H, Hkv=w.Hkv, hd=w.hd, eps=w.rms_eps, mode=mode), W


def inputs(w: Workload):
    plens = draw_prefix_lengths(w)
    return plens, draw_inv_temp(w), kv_provider(w, plens)
