"""Staging of the synthetic inputs into device memory (torch tensors).  No method arithmetic.

bf16 storage is moved as its bit patterns (viewed as torch.bfloat16), so the device holds
exactly the values the oracle reads.
"""
from __future__ import annotations

import concurrent.futures as cf
from typing import Dict, List, Sequence, Tuple

import numpy as np

from .gen import TowerInputs, draw_prefix_kv, _workers
from .workloads import Workload


def _torch():
    import torch
    return torch


def host_to_device(a: np.ndarray, bf16: bool, device="cuda"):
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16) if bf16 else \
        torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def tower_to_device(tw: TowerInputs, device="cuda") -> Dict:
    bf = tw.is_bf16
    up = lambda a: host_to_device(a, bf, device)  # noqa: E731
    upn = lambda a: None if a is None else up(a)  # noqa: E731  (context tower: no pos/final/head)
    # A mixture-of-experts denoiser has no dense MLP: w1/w2 None.
    return dict(tok_emb=up(tw.tok_emb), pos_emb=upn(tw.pos_emb), final_norm=upn(tw.final_norm), lm_head=upn(tw.lm_head),
                attn_norm=[up(a) for a in tw.attn_norm], mlp_norm=[up(a) for a in tw.mlp_norm],
                wq=[up(a) for a in tw.wq], wk=[up(a) for a in tw.wk], wv=[up(a) for a in tw.wv],
                wo=[up(a) for a in tw.wo], w1=[up(a) for a in tw.w1] if tw.w1 else None,
                w2=[up(a) for a in tw.w2] if tw.w2 else None)


def moe_to_device(mi, device="cuda") -> Dict:
    """Expert weights as the binding's set_moe expects them (per-layer lists)."""
    bf = mi.w.dtype == "bf16"
    up = lambda a: host_to_device(a, bf, device)  # noqa: E731
    S = mi.w.moe[2]
    return dict(router=[up(a) for a in mi.router], w1=[up(a) for a in mi.w1], w2=[up(a) for a in mi.w2],
                shared_w1=[up(a) for a in mi.sw1] if S else None, shared_w2=[up(a) for a in mi.sw2] if S else None)


def moe_config(w: Workload) -> Dict:
    E, k, S, de = w.moe
    return dict(n_experts=E, top_k=k, n_shared=S, d_expert=de)


def tower_config(w: Workload, max_batch: int = None, max_prefix_tokens: int = 0) -> Dict:
    return dict(n_layers=w.L, d_model=w.d, n_heads=w.H, n_kv_heads=w.Hkv, head_dim=w.hd, d_ff=w.F, vocab=w.V,
                block_size=w.B, max_batch=max_batch or w.n, max_prefix_tokens=int(max_prefix_tokens),
                dtype=w.dtype, rms_eps=w.rms_eps)


KV_PAGE = 32   # tokens per prefix-cache page


def page_prefix(k: np.ndarray, v: np.ndarray, page: int = KV_PAGE):
    """Natural [P][Hkv][hd] keys/values -> cache pages (the layout of include/td.h).

    V pages: [pages][Hkv][hd][page] (transposed).  K pages: [pages][Hkv][hd/32][2][16][32],
    where slot s of a page sits in half (s // 4) % 2, row (s // 8) * 4 + s % 4.  Pure data
    movement; slots past P in the last page are zero.
    """
    P, Hkv, hd = k.shape
    npg = (P + page - 1) // page
    kp = np.zeros((npg * page, Hkv, hd), dtype=k.dtype)
    vp = np.zeros((npg * page, Hkv, hd), dtype=v.dtype)
    kp[:P], vp[:P] = k, v
    vp = vp.reshape(npg, page, Hkv, hd).transpose(0, 2, 3, 1)
    # slot s = 8 * a + 4 * half + r  ->  (half, row = 4 * a + r)
    kp = kp.reshape(npg, page // 8, 2, 4, Hkv, hd // 32, 32)          # [pg][a][half][r][h][c][e]
    kp = kp.transpose(0, 4, 5, 2, 1, 3, 6).reshape(npg, Hkv, hd // 32, 2, 16, 32)
    return np.ascontiguousarray(kp), np.ascontiguousarray(vp)


def cache_pages(plens: Sequence[int], room: int = 0) -> List[int]:
    """Pages reserved per sequence: its prefix plus `room` more tokens."""
    return [(int(p) + int(room) + KV_PAGE - 1) // KV_PAGE for p in plens]


def prefix_to_device(w: Workload, plens: Sequence[int], device="cuda", layers: int = None, room: int = 0
                     ) -> Tuple[List[int], List, List]:
    """Per-layer paged prefix caches for a batch with prefix lengths plens.

    Returns (token offsets [n+1], K caches, V caches); sequence s owns cache_pages(plens,
    room)[s] consecutive pages (its prefix, then room for `room` appended tokens) starting
    after the pages of sequences 0..s-1.
    """
    torch = _torch()
    offsets = [0]
    for p in plens:
        offsets.append(offsets[-1] + int(p))
    page_off = [0]
    for c in cache_pages(plens, room):
        page_off.append(page_off[-1] + c)
    npages = max(page_off[-1], 1)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    bf = w.dtype == "bf16"
    L = w.L if layers is None else layers
    ks, vs = [], []
    with cf.ThreadPoolExecutor(_workers()) as pool:
        for l in range(L):
            kt = torch.zeros((npages, w.Hkv, w.hd // 32, 2, 16, 32), dtype=dt, device=device)
            vt = torch.zeros((npages, w.Hkv, w.hd, KV_PAGE), dtype=dt, device=device)
            for s, P in enumerate(plens):
                if P == 0:
                    continue
                k = draw_prefix_kv(w, l, s, int(P), "k", pool=pool)
                v = draw_prefix_kv(w, l, s, int(P), "v", pool=pool)
                kp, vp = page_prefix(k, v)
                n_pg = kp.shape[0]
                kt[page_off[s]:page_off[s] + n_pg] = host_to_device(kp, bf, device)
                vt[page_off[s]:page_off[s] + n_pg] = host_to_device(vp, bf, device)
            ks.append(kt)
            vs.append(vt)
    return offsets, ks, vs
