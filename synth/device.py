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
    return dict(tok_emb=up(tw.tok_emb), pos_emb=up(tw.pos_emb), final_norm=up(tw.final_norm), lm_head=up(tw.lm_head),
                attn_norm=[up(a) for a in tw.attn_norm], mlp_norm=[up(a) for a in tw.mlp_norm],
                wq=[up(a) for a in tw.wq], wk=[up(a) for a in tw.wk], wv=[up(a) for a in tw.wv],
                wo=[up(a) for a in tw.wo], w1=[up(a) for a in tw.w1], w2=[up(a) for a in tw.w2])


def tower_config(w: Workload, max_batch: int = None, max_prefix_tokens: int = 0) -> Dict:
    return dict(n_layers=w.L, d_model=w.d, n_heads=w.H, n_kv_heads=w.Hkv, head_dim=w.hd, d_ff=w.F, vocab=w.V,
                block_size=w.B, max_batch=max_batch or w.n, max_prefix_tokens=int(max_prefix_tokens),
                dtype=w.dtype, rms_eps=w.rms_eps)


def prefix_to_device(w: Workload, plens: Sequence[int], device="cuda", layers: int = None
                     ) -> Tuple[List[int], List, List]:
    """Packed per-layer caches [sumP][Hkv][hd] for a batch with prefix lengths plens."""
    torch = _torch()
    offsets = [0]
    for p in plens:
        offsets.append(offsets[-1] + int(p))
    total = offsets[-1]
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    L = w.L if layers is None else layers
    ks, vs = [], []
    with cf.ThreadPoolExecutor(_workers()) as pool:
        for l in range(L):
            kt = torch.empty((max(total, 1), w.Hkv, w.hd), dtype=dt, device=device)
            vt = torch.empty((max(total, 1), w.Hkv, w.hd), dtype=dt, device=device)
            for s, P in enumerate(plens):
                if P == 0:
                    continue
                for which, dst in (("k", kt), ("v", vt)):
                    a = draw_prefix_kv(w, l, s, int(P), which, pool=pool)
                    dst[offsets[s]:offsets[s + 1]] = host_to_device(a, w.dtype == "bf16", device)
            ks.append(kt)
            vs.append(vt)
    return offsets, ks, vs
