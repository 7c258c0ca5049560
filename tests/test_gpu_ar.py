"""GPU parity of the AR decoding mode (td_ar_step on a ctx with block size 1) and of the
denoiser at block size 1.

AR steps are teacher-forced: the oracle's context tower follows the GPU's tokens, and
every GPU prediction must equal the oracle's argmax of that step's logits, except where
the oracle's two largest logits are within 1e-3 of the largest magnitude (a near tie,
after which the comparison stops).  The K/V the steps append must equal the oracle's at
the cache's precision (bf16: at most one rounding apart).
"""
import numpy as np
import pytest

from tests.gpu_common import log

pytestmark = pytest.mark.gpu

CASES = {
    "f32_n2": dict(n=2, plen=("uniform", 0, 40), B=1, d=256, H=4, Hkv=2, hd=64, L=2, F=1024, V=4096, dtype="f32"),
    "bf16_n3": dict(n=3, plen=("uniform", 1, 70), B=1, d=256, H=4, Hkv=4, hd=64, L=2, F=1024, V=4096, dtype="bf16"),
}
STEPS = 6


class AR:
    pass


@pytest.fixture(scope="module", params=sorted(CASES) + ["b1_p4096"])
def ar(request):
    import torch

    from block_diffusion_lm_step_amd import Denoiser
    from oracle import OracleContextTower, OracleTower
    from synth import Workload, draw_inv_temp, draw_prefix_lengths, draw_tower, get_workload
    from synth.device import cache_pages, prefix_to_device, tower_config, tower_to_device
    from tests.helpers import kv_provider, oracle_weights

    m = AR()
    if request.param in CASES:
        m.w = w = Workload(name=request.param, tower="ar_" + request.param, weight_std=0.02, **CASES[request.param])
        m.steps = STEPS
    else:   # the single-sequence 4096-prefix tower at block size 1
        m.w = w = get_workload(request.param).with_(B=1)
        m.steps = 3
    log(f"[ar] building {w.name}")
    tw, tc = draw_tower(w), draw_tower(w, context=True, ar_head=True)
    m.plens = draw_prefix_lengths(w)
    m.tau = draw_inv_temp(w)
    m.kv = kv_provider(w, m.plens)
    m.caps = cache_pages(m.plens, m.steps)
    m.page_off = np.concatenate([[0], np.cumsum(m.caps)]).astype(int)
    _, m.ks, m.vs = prefix_to_device(w, m.plens, room=m.steps)
    m.dev = Denoiser(tower_config(w, max_batch=w.n, max_prefix_tokens=int(m.plens.sum()) + m.steps * w.n),
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


def test_denoiser_block_of_one(ar):
    """Block size 1: one step adopts the single position's prediction (oracle loop, B = 1)."""
    from oracle import oracle_generate
    w, torch = ar.w, ar.torch
    tok_o, cs_o, st_o, _ = oracle_generate(ar.orc, w.n, 1, ar.tau, w.gamma, ar.kv, keep_trace=False)
    tok = torch.zeros((w.n, 1), dtype=torch.int32, device="cuda")
    com = torch.zeros((w.n, 1), dtype=torch.uint8, device="cuda")
    steps = torch.zeros(w.n, dtype=torch.int32, device="cuda")
    ar.dev.generate_block(tok, com, ar.tau_d, w.gamma, steps=steps)
    ar.dev.sync()
    assert np.array_equal(tok.cpu().numpy(), tok_o) and (steps.cpu().numpy() == 1).all()


def test_ar_decode_teacher_forced(ar):
    from oracle import round_bf16
    w, torch = ar.w, ar.torch
    bf = w.dtype == "bf16"
    added = {}

    def kv_now(l, s):
        K, V = ar.kv(l, s)
        e = added.get((l, s), [])
        if not e:
            return K, V
        return (np.concatenate([np.asarray(K, np.float64)] + [x[0] for x in e]),
                np.concatenate([np.asarray(V, np.float64)] + [x[1] for x in e]))

    cur = np.arange(w.n, dtype=np.int64) * 7 + 3
    tok = torch.from_numpy(cur.astype(np.int32)).cuda()
    agree = 0
    for t in range(ar.steps):
        kvs, z = ar.ctx.ar_step(cur, kv_now, range(w.n))
        for l, (k, v) in enumerate(kvs):
            for s in range(w.n):
                added.setdefault((l, s), []).append((round_bf16(k[s]), round_bf16(v[s])) if bf else (k[s], v[s]))
        ar.dev.ar_step(tok)
        ar.dev.sync()
        g = tok.cpu().numpy().astype(np.int64)
        want = np.argmax(z.astype(np.float32), axis=1)
        top2 = np.sort(z, axis=1)[:, -2:]
        near = (top2[:, 1] - top2[:, 0]) < 1e-3 * np.abs(z).max(axis=1)
        bad = (g != want) & ~near
        log(f"[{w.name}] AR step {t}: gpu {g.tolist()} oracle {want.tolist()} near-tie {near.tolist()}")
        assert not bad.any(), (t, g, want)
        if (g != want).any():
            break   # a near tie went the other way: the runs diverge from here
        agree += 1
        cur = g
    assert agree >= 1
    # the appended cache entries of the agreed steps
    worst = 0.0
    for l in range(w.L):
        kt, vt = ar.ks[l].float().cpu().numpy(), ar.vs[l].float().cpu().numpy()
        for s in range(w.n):
            P = int(ar.plens[s])
            for i in range(agree):
                t = P + i
                pg, slot = ar.page_off[s] + t // 32, t % 32
                half, row = (slot // 4) % 2, (slot // 8) * 4 + slot % 4
                kg = kt[pg, :, :, half, row, :].reshape(w.Hkv, w.hd)
                vg = vt[pg, :, :, slot]
                ko, vo = added[(l, s)][i]
                for gg, oo in ((kg, ko), (vg, vo)):
                    err = np.abs(gg - oo) / np.abs(oo).max(axis=-1, keepdims=True)
                    worst = max(worst, float(err.max()))
                    assert err.max() <= (2.0 ** -7 if bf else 1e-4)
    log(f"[{w.name}] {agree} AR steps agreed; appended K/V worst relative error {worst:.2e}")
