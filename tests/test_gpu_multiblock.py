"""GPU parity of multi-block generation: td_generate_block, then td_append_block (the
frozen context tower's causal pass over the block and the K/V append into caches bound
with room), repeated for three blocks on small towers and two at full size (batch 1, prefix 4096).

Every block of every sequence is compared with the oracle's multi-block loop: tokens,
commit steps and step counts exactly.  The appended cache entries are compared with the
oracle context tower's K/V at the cache's precision (bf16: at most one rounding apart,
nearly all identical; fp32: 1e-4 of the row's largest value), and the pages outside the
appended slots must be unchanged.
"""
import numpy as np
import pytest

from tests.gpu_common import log

pytestmark = pytest.mark.gpu

N_BLOCKS = 3
CASES = {
    "f32_n2_b16": dict(n=2, plen=("uniform", 0, 40), B=16, d=256, H=4, Hkv=2, hd=64, L=2, F=1024, V=4096,
                       dtype="f32"),
    "bf16_n3_b16": dict(n=3, plen=("uniform", 0, 70), B=16, d=256, H=4, Hkv=2, hd=64, L=2, F=1024, V=4096,
                        dtype="bf16"),
    # R = G * B = 128 query rows per K/V head: the grouped-query attention path, causal block keys in the first item.
    "bf16_n2_b32_gqa": dict(n=2, plen=("uniform", 1, 50), B=32, d=256, H=8, Hkv=2, hd=64, L=2, F=1024, V=4096,
                            dtype="bf16"),
    # Grouped-query pairs with no prefix at all: the empty prefix item that appended blocks extend.
    "bf16_n2_b32_gqa_empty": dict(n=2, plen=("fixed", 0), B=32, d=256, H=8, Hkv=2, hd=64, L=2, F=1024, V=4096,
                                  dtype="bf16"),
    # Prefixes of ~490 tokens (split-K chunks of 256): the last chunk grows by 32 per block and
    # passes twice the chunk size at the ninth block, where the work lists are rebuilt.
    "bf16_n2_b32_grow": dict(n=2, plen=("uniform", 480, 500), B=32, d=256, H=4, Hkv=4, hd=64, L=2, F=1024, V=4096,
                             dtype="bf16", blocks=10),
}


class MB:
    pass


@pytest.fixture(scope="module", params=sorted(CASES) + ["b1_p4096"])
def mb(request):
    import torch

    from block_diffusion_lm_step_amd import Denoiser
    from oracle import OracleContextTower, OracleTower
    from synth import Workload, draw_inv_temp, draw_prefix_lengths, draw_tower
    from synth.device import cache_pages, prefix_to_device, tower_config, tower_to_device
    from tests.helpers import kv_provider, oracle_weights

    from synth import get_workload
    m = MB()
    if request.param in CASES:
        kw = dict(CASES[request.param])
        m.blocks = kw.pop("blocks", N_BLOCKS)
        m.w = w = Workload(name=request.param, tower="mb_" + request.param, weight_std=0.02, **kw)
    else:   # full size: the single-sequence 4096-prefix workload, two blocks
        m.w = w = get_workload(request.param)
        m.blocks = 2
    log(f"[mb] building {w.name}")
    tw, tc = draw_tower(w), draw_tower(w, context=True)
    m.plens = draw_prefix_lengths(w)
    m.tau = draw_inv_temp(w)
    m.kv = kv_provider(w, m.plens)
    room = m.blocks * w.B
    m.caps = cache_pages(m.plens, room)
    m.page_off = np.concatenate([[0], np.cumsum(m.caps)]).astype(int)
    _, m.ks, m.vs = prefix_to_device(w, m.plens, room=room)
    m.dev = Denoiser(tower_config(w, max_batch=w.n, max_prefix_tokens=int(m.plens.sum()) + room * w.n),
                     tower_to_device(tw))
    m.dev.bind_cache(m.plens.tolist(), m.caps, m.ks, m.vs)
    m.dev.set_context_tower(tower_to_device(tc))
    m.orc = OracleTower(oracle_weights(tw), H=w.H, Hkv=w.Hkv, hd=w.hd, eps=w.rms_eps, mode="plain")
    m.ctx = OracleContextTower(oracle_weights(tc), H=w.H, Hkv=w.Hkv, hd=w.hd, eps=w.rms_eps)
    m.torch = torch
    m.tau_d = torch.from_numpy(m.tau).cuda()
    torch.cuda.synchronize()
    yield m
    m.dev.close()


def _unpage(w, kt, vt, page0, t0, t1):
    """Natural [t1-t0][Hkv][hd] keys and values of tokens t0..t1-1 of the sequence whose
    pages start at page0 (the cache layout of include/td.h; pure data movement)."""
    k = np.empty((t1 - t0, w.Hkv, w.hd), np.float32)
    v = np.empty((t1 - t0, w.Hkv, w.hd), np.float32)
    for i, t in enumerate(range(t0, t1)):
        pg, slot = page0 + t // 32, t % 32
        half, row = (slot // 4) % 2, (slot // 8) * 4 + slot % 4
        k[i] = kt[pg, :, :, half, row, :].reshape(w.Hkv, w.hd)
        v[i] = vt[pg, :, :, slot]
    return k, v


def test_generate_and_append_blocks(mb):
    from oracle import oracle_generate_blocks
    w, torch = mb.w, mb.torch
    bf = w.dtype == "bf16"
    nb = mb.blocks
    toks_o, cs_o, st_o, added = oracle_generate_blocks(mb.orc, mb.ctx, nb, w.n, w.B, mb.tau, w.gamma, mb.kv,
                                                      cache_bf16=bf, return_kv=True)
    before = [(k.float().cpu().numpy().copy(), v.float().cpu().numpy().copy()) for k, v in zip(mb.ks, mb.vs)]
    for b in range(nb):
        tok = torch.zeros((w.n, w.B), dtype=torch.int32, device="cuda")
        com = torch.zeros((w.n, w.B), dtype=torch.uint8, device="cuda")
        steps = torch.zeros(w.n, dtype=torch.int32, device="cuda")
        cstep = torch.zeros((w.n, w.B), dtype=torch.int8, device="cuda")
        mb.dev.generate_block(tok, com, mb.tau_d, w.gamma, steps=steps, commit_step=cstep)
        mb.dev.sync()
        tg, cg, sg = tok.cpu().numpy(), cstep.cpu().numpy(), steps.cpu().numpy()
        log(f"[{w.name}] block {b}: steps gpu {sg} oracle {st_o[b]}; tokens equal {np.array_equal(tg, toks_o[b])}")
        assert np.array_equal(tg, toks_o[b]) and np.array_equal(cg, cs_o[b]) and np.array_equal(sg, st_o[b])
        mb.dev.append_block(tok)
        mb.dev.sync()
    # appended entries against the oracle context tower; everything else unchanged
    worst, same, total = 0.0, 0, 0
    for l in range(w.L):
        kt, vt = mb.ks[l].float().cpu().numpy(), mb.vs[l].float().cpu().numpy()
        for s in range(w.n):
            P = int(mb.plens[s])
            kg, vg = _unpage(w, kt, vt, mb.page_off[s], P, P + nb * w.B)
            ko = np.concatenate([e[0] for e in added[(l, s)]])
            vo = np.concatenate([e[1] for e in added[(l, s)]])
            for g, o in ((kg, ko), (vg, vo)):
                scale = np.abs(o).max(axis=-1, keepdims=True)
                err = np.abs(g.astype(np.float64) - o) / scale
                worst = max(worst, float(err.max()))
                same += int((g == o.astype(np.float32)).sum())
                total += g.size
                assert err.max() <= (2.0 ** -7 if bf else 1e-4), (l, s, float(err.max()))
            kb, vb = _unpage(w, before[l][0], before[l][1], mb.page_off[s], 0, P)
            ka, va = _unpage(w, kt, vt, mb.page_off[s], 0, P)
            assert np.array_equal(ka, kb) and np.array_equal(va, vb), "prefix entries changed"
        # pages of no sequence's tokens (the slack after each sequence's tokens) untouched
        for s in range(w.n):
            end_tok = int(mb.plens[s]) + nb * w.B
            first_free = mb.page_off[s] + (end_tok + 31) // 32
            assert np.array_equal(kt[first_free:mb.page_off[s + 1]], before[l][0][first_free:mb.page_off[s + 1]])
    log(f"[{w.name}] appended K/V: worst relative error {worst:.2e}, identical {same}/{total}")
    if bf:
        assert same >= 0.99 * total


def test_append_block_errors(mb):
    """Refused before anything runs: a binding with no room for B more tokens (one
    sequence of 32 tokens in one page), and a ctx with no context tower."""
    from block_diffusion_lm_step_amd import Denoiser, TdError
    from synth import draw_tower
    from synth.device import tower_config, tower_to_device
    w, torch = mb.w, mb.torch
    tok = torch.zeros((1, w.B), dtype=torch.int32, device="cuda")
    mb.dev.bind_cache([32], [1], mb.ks, mb.vs)
    with pytest.raises(TdError, match="no room"):
        mb.dev.append_block(tok)
    dev2 = Denoiser(tower_config(w, max_batch=1, max_prefix_tokens=64), tower_to_device(draw_tower(w)))
    try:
        dev2.bind_cache([0], [2], mb.ks, mb.vs)
        with pytest.raises(TdError, match="no context tower"):
            dev2.append_block(tok)
    finally:
        dev2.close()
