"""Keyed, chunked draws of every synthetic input.

Stream key: SeedSequence([seed, owner, tensor_id, layer, seq, chunk]) where `owner`
is a stable integer of the tower name (weights) or the batch name (prefix lengths,
prefix K/V, inverse temperatures).  A tensor is cut into chunks of CHUNK elements
in row-major order and each chunk has its own stream, so a slice regenerates
identically whatever the thread count or the slice boundaries.

Storage: float32 workloads store float32; bfloat16 workloads store uint16 bit
patterns obtained from the float32 draw by round-to-nearest-even.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import os
import zlib
from typing import Dict, List, Optional

import numpy as np

from .workloads import Workload

CHUNK = 1 << 22

T_TOK_EMB, T_POS_EMB = 1, 2
T_WQ, T_WK, T_WV, T_WO, T_W1, T_W2 = 10, 11, 12, 13, 14, 15
T_LM_HEAD = 20
T_MOE_ROUTER, T_MOE_W1, T_MOE_W2, T_MOE_SW1, T_MOE_SW2 = 16, 17, 18, 19, 21
T_PREFIX_K, T_PREFIX_V = 30, 31
T_INV_TEMP, T_PREFIX_LEN = 40, 41


def _owner(name: str) -> int:
    return zlib.crc32(name.encode()) & 0x7FFFFFFF


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _fill_normal(out_flat: np.ndarray, start: int, stop: int, key: List[int], std: float,
                 as_bf16: bool) -> None:
    """Fill out_flat[start:stop] (element indices of the whole tensor) chunk by chunk."""
    c0, c1 = start // CHUNK, (stop - 1) // CHUNK
    for c in range(c0, c1 + 1):
        lo, hi = max(start, c * CHUNK), min(stop, (c + 1) * CHUNK)
        rng = np.random.default_rng(np.random.SeedSequence(key + [c]))
        # A chunk always draws from its first element (the stream's values are sequential),
        # so a partial chunk agrees with the same elements of a whole one.
        vals = rng.standard_normal(hi - c * CHUNK, dtype=np.float32)[lo - c * CHUNK:]
        vals = vals * np.float32(std)
        dst = out_flat[lo - start: hi - start]
        dst[...] = bf16_bits_from_f32(vals) if as_bf16 else vals


def draw_normal(shape, key: List[int], std: float, as_bf16: bool, *, start: int = 0,
                stop: Optional[int] = None, pool: Optional[cf.Executor] = None) -> np.ndarray:
    """Elements [start, stop) of a keyed N(0, std^2) tensor of `shape` (flattened row-major)."""
    total = int(np.prod(shape))
    stop = total if stop is None else stop
    out = np.empty(stop - start, dtype=np.uint16 if as_bf16 else np.float32)
    bounds = list(range(start - start % CHUNK, stop, CHUNK))
    pieces = [(max(start, b), min(stop, b + CHUNK)) for b in bounds]
    pieces = [(a, b) for a, b in pieces if a < b]

    def work(ab):
        a, b = ab
        _fill_normal(out[a - start: b - start], a, b, key, std, as_bf16)

    if len(pieces) > 1:
        own = pool is None
        ex = pool or cf.ThreadPoolExecutor(_workers())
        try:
            list(ex.map(work, pieces))
        finally:
            if own:
                ex.shutdown()
    else:
        for p in pieces:
            work(p)
    if start == 0 and stop == total:
        return out.reshape(shape)
    return out


@dataclasses.dataclass
class TowerInputs:
    """Weights of one denoiser tower, row-major [out][in], in their storage dtype.

    tok_emb is [V+1][d]; row V is the [MASK] embedding.  pos_emb is [B][d], one learned
    row per block position.  Norm gains are ones.
    """
    w: Workload
    tok_emb: np.ndarray
    pos_emb: np.ndarray
    wq: List[np.ndarray]
    wk: List[np.ndarray]
    wv: List[np.ndarray]
    wo: List[np.ndarray]
    w1: List[np.ndarray]
    w2: List[np.ndarray]
    attn_norm: List[np.ndarray]
    mlp_norm: List[np.ndarray]
    final_norm: np.ndarray
    lm_head: np.ndarray

    @property
    def is_bf16(self) -> bool:
        return self.w.dtype == "bf16"

    def as_f32(self, a: np.ndarray) -> np.ndarray:
        """Exact float32 view of a stored value array (bf16 bits are widened exactly)."""
        return f32_from_bf16_bits(a) if self.is_bf16 else np.asarray(a, dtype=np.float32)

    def layer_arrays(self, l: int) -> Dict[str, np.ndarray]:
        return dict(wq=self.wq[l], wk=self.wk[l], wv=self.wv[l], wo=self.wo[l], w1=self.w1[l],
                    w2=self.w2[l], attn_norm=self.attn_norm[l], mlp_norm=self.mlp_norm[l])


def draw_tower(w: Workload, *, layers: Optional[int] = None, context: bool = False,
               ar_head: bool = False) -> TowerInputs:
    """Draw the tower weights of workload `w` (optionally only its first `layers` layers).

    context=True draws the frozen context tower that writes the prefix cache: the same
    shapes from streams of its own (owner "<tower>/context"); it has no position table,
    and no final norm or LM head unless ar_head=True (the AR decoding mode).
    """
    bf = w.dtype == "bf16"
    own = _owner(w.tower + "/context" if context else w.tower)
    std = w.weight_std
    L = w.L if layers is None else layers
    with cf.ThreadPoolExecutor(_workers()) as ex:
        def nrm(shape, tid, layer=0, seq=0):
            return draw_normal(shape, [w.seed, own, tid, layer, seq], std, bf, pool=ex)

        tok_emb = nrm((w.V + 1, w.d), T_TOK_EMB)
        pos_emb = None if context else nrm((w.B, w.d), T_POS_EMB, layer=w.B)
        wq = [nrm((w.H * w.hd, w.d), T_WQ, l) for l in range(L)]
        wk = [nrm((w.Hkv * w.hd, w.d), T_WK, l) for l in range(L)]
        wv = [nrm((w.Hkv * w.hd, w.d), T_WV, l) for l in range(L)]
        wo = [nrm((w.d, w.H * w.hd), T_WO, l) for l in range(L)]
        dense = not (w.moe and not context)   # a mixture-of-experts denoiser has no dense MLP
        w1 = [nrm((w.F, w.d), T_W1, l) for l in range(L)] if dense else []
        w2 = [nrm((w.d, w.F), T_W2, l) for l in range(L)] if dense else []
        lm_head = None if context and not ar_head else nrm((w.V, w.d), T_LM_HEAD)
    one = bf16_bits_from_f32(np.ones(w.d, np.float32)) if bf else np.ones(w.d, np.float32)
    return TowerInputs(w=w, tok_emb=tok_emb, pos_emb=pos_emb, wq=wq, wk=wk, wv=wv, wo=wo, w1=w1, w2=w2,
                       attn_norm=[one.copy() for _ in range(L)], mlp_norm=[one.copy() for _ in range(L)],
                       final_norm=None if context and not ar_head else one.copy(), lm_head=lm_head)


@dataclasses.dataclass
class MoeInputs:
    """Mixture-of-experts weights of a denoiser, per layer, in the storage dtype:
    router [E][d], w1 [E][d_expert][d], w2 [E][d][d_expert], sw1 [n_shared][d_expert][d],
    sw2 [n_shared][d][d_expert]."""
    w: Workload
    router: List[np.ndarray]
    w1: List[np.ndarray]
    w2: List[np.ndarray]
    sw1: List[np.ndarray]
    sw2: List[np.ndarray]


def draw_moe(w: Workload, *, layers: Optional[int] = None) -> MoeInputs:
    """Draw the expert weights of workload `w` (N(0, weight_std^2), like the other weights)."""
    if not w.moe:
        raise ValueError(f"workload {w.name} has no mixture of experts")
    E, _, S, de = w.moe
    bf = w.dtype == "bf16"
    own = _owner(w.tower)
    L = w.L if layers is None else layers
    with cf.ThreadPoolExecutor(_workers()) as ex:
        def nrm(shape, tid, layer):
            return draw_normal(shape, [w.seed, own, tid, layer, 0], w.weight_std, bf, pool=ex)

        router = [nrm((E, w.d), T_MOE_ROUTER, l) for l in range(L)]
        w1 = [nrm((E, de, w.d), T_MOE_W1, l) for l in range(L)]
        w2 = [nrm((E, w.d, de), T_MOE_W2, l) for l in range(L)]
        sw1 = [nrm((S, de, w.d), T_MOE_SW1, l) for l in range(L)]
        sw2 = [nrm((S, w.d, de), T_MOE_SW2, l) for l in range(L)]
    return MoeInputs(w=w, router=router, w1=w1, w2=w2, sw1=sw1, sw2=sw2)


def draw_prefix_lengths(w: Workload) -> np.ndarray:
    """int64 [n] prefix lengths: fixed, or uniform integers with both bounds inclusive."""
    if w.plen[0] == "fixed":
        return np.full(w.n, int(w.plen[1]), dtype=np.int64)
    lo, hi = int(w.plen[1]), int(w.plen[2])
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, _owner(w.batch), T_PREFIX_LEN, 0, 0]))
    return rng.integers(lo, hi, endpoint=True, size=w.n).astype(np.int64)


def draw_inv_temp(w: Workload) -> np.ndarray:
    """float32 [n][B] per-position logit inverse temperature, log-uniform on tau_range."""
    lo, hi = w.tau_range
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, _owner(w.batch), T_INV_TEMP, w.B, 0]))
    u = rng.random((w.n, w.B))
    return np.exp(np.log(lo) + u * (np.log(hi) - np.log(lo))).astype(np.float32)


def draw_prefix_kv(w: Workload, layer: int, seq: int, P: int, which: str, *, tok_start: int = 0,
                   tok_stop: Optional[int] = None, pool: Optional[cf.Executor] = None) -> np.ndarray:
    """Prefix keys or values of (layer, seq): tokens [tok_start, tok_stop) as [T][Hkv][hd]."""
    tid = T_PREFIX_K if which == "k" else T_PREFIX_V
    row = w.Hkv * w.hd
    tok_stop = P if tok_stop is None else tok_stop
    flat = draw_normal((P, w.Hkv, w.hd), [w.seed, _owner(w.batch), tid, layer, seq], w.kv_std,
                       w.dtype == "bf16", start=tok_start * row, stop=tok_stop * row, pool=pool)
    return flat.reshape(tok_stop - tok_start, w.Hkv, w.hd)
