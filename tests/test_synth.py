"""The seeded input generator: determinism, chunk independence, bf16 encoding, ranges."""
import numpy as np
import pytest
import torch

from synth import (WORKLOADS, bf16_bits_from_f32, draw_inv_temp, draw_prefix_kv, draw_prefix_lengths,
                   draw_tower, f32_from_bf16_bits, get_workload)
from synth.gen import CHUNK, draw_normal


def test_chunked_slices_match_whole_draw():
    shape = (3 * CHUNK + 17,)
    whole = draw_normal(shape, [0, 7, 1, 2, 3], 0.5, False)
    for lo, hi in [(0, 5), (CHUNK - 3, CHUNK + 3), (CHUNK + 1, 3 * CHUNK + 17), (2 * CHUNK, 2 * CHUNK + 1)]:
        part = draw_normal(shape, [0, 7, 1, 2, 3], 0.5, False, start=lo, stop=hi)
        assert np.array_equal(whole[lo:hi], part)


def test_keys_give_independent_streams():
    a = draw_normal((1000,), [0, 1, 2, 3, 4], 1.0, False)
    b = draw_normal((1000,), [0, 1, 2, 3, 5], 1.0, False)
    assert not np.array_equal(a, b)
    assert np.array_equal(a, draw_normal((1000,), [0, 1, 2, 3, 4], 1.0, False))
    assert abs(a.std() - 1.0) < 0.1


def test_bf16_encoding_matches_torch_rne():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # exact ties: low 16 bits == 0x8000 under every kept 7-bit mantissa, both signs
    ties = ((rng.integers(0, 1 << 7, 2000, dtype=np.uint32) << 16) | np.uint32(0x8000)
            | (rng.integers(0, 2, 2000, dtype=np.uint32) << 31) | np.uint32(0x3F000000))
    x = np.concatenate([x, ties.view(np.float32), np.array([0.0, -0.0, 1e-40, -3e-39], np.float32)])
    ours = bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(f32_from_bf16_bits(ours), torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16)
                          .float().numpy())


def test_prefix_lengths_and_inverse_temperature_ranges():
    w = WORKLOADS["ragged32"]
    p = draw_prefix_lengths(w)
    assert p.shape == (32,) and p.min() >= 512 and p.max() <= 8192
    assert np.array_equal(p, draw_prefix_lengths(w))
    assert (draw_prefix_lengths(WORKLOADS["gqa_long"]) == 65536).all()
    tau = draw_inv_temp(WORKLOADS["sweep64_b32"])
    assert tau.shape == (64, 32) and tau.dtype == np.float32
    assert tau.min() >= 1.0 and tau.max() < 64.0
    # log-uniform: log(tau)/log(64) is roughly uniform
    u = np.log(tau.astype(np.float64)) / np.log(64.0)
    assert abs(u.mean() - 0.5) < 0.05
    # sweep workloads share their batch (prefix lengths) across block sizes
    assert np.array_equal(draw_prefix_lengths(WORKLOADS["sweep64_b8"]), draw_prefix_lengths(WORKLOADS["sweep64_b32"]))


def test_tower_shapes_and_storage():
    w = get_workload("tiny_fp32")
    tw = draw_tower(w)
    assert tw.tok_emb.shape == (w.V + 1, w.d) and tw.tok_emb.dtype == np.float32
    assert tw.pos_emb.shape == (w.B, w.d)
    assert tw.wq[0].shape == (w.H * w.hd, w.d) and tw.wk[0].shape == (w.Hkv * w.hd, w.d)
    assert tw.wo[0].shape == (w.d, w.H * w.hd) and tw.w1[0].shape == (w.F, w.d) and tw.w2[0].shape == (w.d, w.F)
    assert tw.lm_head.shape == (w.V, w.d)
    assert (tw.attn_norm[0] == 1).all() and (tw.final_norm == 1).all()
    assert abs(float(tw.w1[0].std()) - 0.02) < 1e-3
    bw = get_workload("b1_p4096").with_(tower="b1_small", L=1, V=256, d=128, F=512, H=2, Hkv=2)
    btw = draw_tower(bw)
    assert btw.wq[0].dtype == np.uint16
    assert (f32_from_bf16_bits(btw.attn_norm[0]) == 1).all()


def test_moe_weights_shapes_streams_and_storage():
    from synth import draw_moe
    w = get_workload("tiny_fp32").with_(tower="tiny_moe", moe=(8, 2, 1, 64))
    mi = draw_moe(w)
    E, k, S, de = w.moe
    assert len(mi.router) == w.L and mi.router[0].shape == (E, w.d)
    assert mi.w1[0].shape == (E, de, w.d) and mi.w2[0].shape == (E, w.d, de)
    assert mi.sw1[0].shape == (S, de, w.d) and mi.sw2[0].shape == (S, w.d, de)
    assert abs(float(mi.w1[0].std()) - 0.02) < 2e-3
    # keyed streams: the same draw twice, different tensors and layers differ
    again = draw_moe(w)
    assert np.array_equal(again.w1[1], mi.w1[1]) and np.array_equal(again.router[0], mi.router[0])
    assert not np.array_equal(mi.w1[0][:, :, :64].reshape(-1)[:4096], mi.w2[0].reshape(-1)[:4096])
    assert not np.array_equal(mi.router[0], mi.router[1])
    # a mixture-of-experts tower has no dense MLP; the context tower keeps one
    tw = draw_tower(w)
    assert tw.w1 == [] and tw.w2 == []
    assert draw_tower(w, context=True).w1[0].shape == (w.F, w.d)
    bw = w.with_(dtype="bf16", tower="tiny_moe_bf16")
    assert draw_moe(bw).w2[0].dtype == np.uint16
    with pytest.raises(ValueError):
        draw_moe(get_workload("tiny_fp32"))


def test_prefix_kv_token_slices():
    w = get_workload("tiny_fp32")
    full = draw_prefix_kv(w, 1, 0, 128, "k")
    assert full.shape == (128, w.Hkv, w.hd)
    assert np.array_equal(full[40:77], draw_prefix_kv(w, 1, 0, 128, "k", tok_start=40, tok_stop=77))
    assert not np.array_equal(full, draw_prefix_kv(w, 1, 0, 128, "v"))
    assert abs(full.std() - 1.0) < 0.05


def test_prefix_page_layout_matches_the_documented_offsets():
    """Cache pages as include/td.h states them.  V: ((p*Hkv + h)*hd + e)*32 + s.
    K: (p*Hkv + h)*32*hd + ((e//32)*2 + (s//4)%2)*512 + ((s//8)*4 + s%4)*32 + e%32."""
    from synth.device import KV_PAGE, page_prefix
    rng = np.random.default_rng(4)
    P, Hkv, hd = 77, 3, 64
    k = rng.standard_normal((P, Hkv, hd)).astype(np.float32)
    v = rng.standard_normal((P, Hkv, hd)).astype(np.float32)
    kp, vp = page_prefix(k, v)
    npg = (P + KV_PAGE - 1) // KV_PAGE
    assert kp.size == npg * Hkv * KV_PAGE * hd and vp.shape == (npg, Hkv, hd, KV_PAGE)
    kf, vf = kp.reshape(-1), vp.reshape(-1)

    def koff(p_, h, s, e):
        return (p_ * Hkv + h) * KV_PAGE * hd + ((e // 32) * 2 + (s // 4) % 2) * 512 + ((s // 8) * 4 + s % 4) * 32 + e % 32

    for t in range(P):
        p_, s_ = divmod(t, KV_PAGE)
        for h in range(Hkv):
            for e in (0, 5, 31, 32, 63):
                assert kf[koff(p_, h, s_, e)] == k[t, h, e]
                assert vf[((p_ * Hkv + h) * hd + e) * KV_PAGE + s_] == v[t, h, e]
    # every element appears exactly once (the K map is a bijection on a page)
    offs = {koff(0, 0, s_, e) for s_ in range(KV_PAGE) for e in range(hd)}
    assert offs == set(range(KV_PAGE * hd))
    for s_ in range(P % KV_PAGE, KV_PAGE):   # padding slots of the last page are zero
        for e in range(hd):
            assert kf[koff(npg - 1, 1, s_, e)] == 0 and vf[((npg - 1) * Hkv * hd + hd + e) * KV_PAGE + s_] == 0
