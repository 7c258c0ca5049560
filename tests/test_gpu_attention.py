"""GPU parity of the split-K prefix+block attention (td_debug_attention) against the oracle.

Ragged prefixes (0, 1, not a multiple of the chunk, several chunks), grouped-query head
maps, block sizes 8/16/32, fp32 and bf16, and the long-context GQA shape at full size.
"""
import numpy as np
import pytest

from tests.gpu_common import log

pytestmark = pytest.mark.gpu


def _run(dtype, H, Hkv, hd, B, plens, seed=0, qscale=1.0):
    import torch

    from block_diffusion_lm_step_amd import Denoiser
    from oracle import joint_attention
    from synth import Workload, draw_tower, f32_from_bf16_bits
    from synth.device import KV_PAGE, prefix_to_device, tower_config, tower_to_device
    from synth.gen import draw_prefix_kv

    n = len(plens)
    w = Workload(name=f"attn_{dtype}_{H}_{Hkv}_{hd}_{B}", tower="attn_probe", n=n, plen=("fixed", 0), B=B, d=64,
                 H=H, Hkv=Hkv, hd=hd, L=1, F=64, V=64, dtype=dtype)
    log(f"[attn] dtype={dtype} H={H} Hkv={Hkv} hd={hd} B={B} plens={list(plens)[:8]}{'...' if n > 8 else ''}")
    dW = tower_to_device(draw_tower(w))
    offsets, ks, vs = prefix_to_device(w, plens)
    # The cache contract leaves the slots past a prefix's end undefined: poison them.
    page = 0
    for P in plens:
        npg = (P + KV_PAGE - 1) // KV_PAGE
        for slot in range(P % KV_PAGE if P % KV_PAGE else KV_PAGE, KV_PAGE):
            # K page [Hkv][hd/32][half][row][32]: slot -> half (slot // 4) % 2, row (slot // 8) * 4 + slot % 4
            ks[0][page + npg - 1, :, :, (slot // 4) % 2, (slot // 8) * 4 + slot % 4, :] = float("nan")
            vs[0][page + npg - 1, :, :, slot] = float("nan")
        page += npg
    dev = Denoiser(tower_config(w, max_batch=n, max_prefix_tokens=max(1, offsets[-1])), dW)
    dev.set_prefix(offsets, ks, vs)
    rng = np.random.default_rng(seed)
    Nqkv = (H + 2 * Hkv) * hd
    qkv = (rng.standard_normal((n * B, Nqkv)) * qscale).astype(np.float32)   # fp32 activations
    qkv_d = torch.from_numpy(qkv).cuda()
    o_d = torch.zeros((n * B, H * hd), dtype=torch.float32, device="cuda")
    dev.debug_attention(0, qkv_d, o_d)
    dev.sync()
    o = o_d.cpu().numpy().reshape(n, B, H, hd)
    q3 = qkv.reshape(n, B, Nqkv).astype(np.float64)
    worst = 0.0
    for s in range(n):
        P = int(plens[s])
        k_pre = draw_prefix_kv(w, 0, s, P, "k")
        v_pre = draw_prefix_kv(w, 0, s, P, "v")
        if dtype == "bf16":
            k_pre, v_pre = f32_from_bf16_bits(k_pre), f32_from_bf16_bits(v_pre)
        k_pre, v_pre = k_pre.astype(np.float64), v_pre.astype(np.float64)
        q = q3[s, :, :H * hd].reshape(B, H, hd)
        kb = q3[s, :, H * hd:(H + Hkv) * hd].reshape(B, Hkv, hd)
        vb = q3[s, :, (H + Hkv) * hd:].reshape(B, Hkv, hd)
        ref = joint_attention(q, k_pre, v_pre, kb, vb)
        # fp32 accumulation; with bf16 keys the fp32 queries and probabilities enter the
        # MFMA as hi + lo bf16 parts (relative error <= 2^-17 each)
        assert np.isfinite(o[s]).all(), f"seq {s}: non-finite output"
        err = float(np.abs(o[s] - ref).max() / np.abs(ref).max())
        worst = max(worst, err)
        assert err < (3e-5 if dtype == "bf16" else 1e-5), f"seq {s}: rel err {err:.3e}"
    log(f"[attn] worst relative error {worst:.3e}")
    dev.close()


@pytest.mark.parametrize("plens", [[0], [1], [37], [128], [300, 0, 1, 129, 256]])
def test_fp32_mha_ragged(plens):
    _run("f32", H=4, Hkv=4, hd=64, B=16, plens=plens)


@pytest.mark.parametrize("H,Hkv,B", [(8, 2, 16), (16, 1, 16), (4, 4, 8), (4, 4, 32), (6, 3, 8)])
def test_fp32_gqa_and_block_sizes(H, Hkv, B):
    _run("f32", H=H, Hkv=Hkv, hd=64, B=B, plens=[77, 300, 0])


@pytest.mark.parametrize("H,Hkv,B,plens", [(16, 16, 16, [4096]), (16, 16, 8, [1000, 3]), (16, 16, 32, [2047, 0]),
                                           (32, 2, 16, [5000, 1]), (12, 1, 16, [700, 33, 0])])
def test_bf16_shapes(H, Hkv, B, plens):
    _run("bf16", H=H, Hkv=Hkv, hd=128, B=B, plens=plens, qscale=0.5)


@pytest.mark.parametrize("H,Hkv,B,plens", [(8, 2, 16, [777, 40, 0]), (16, 1, 16, [300, 1])])
def test_bf16_gqa_head_dim_64(H, Hkv, B, plens):
    """Grouped-query rows at head size 64: half of the workgroup's threads stage no chunk."""
    _run("bf16", H=H, Hkv=Hkv, hd=64, B=B, plens=plens, qscale=0.5)


def test_bf16_long_context_gqa_full_size():
    """4 sequences x 65536 prefix keys, 32 query heads over 2 K/V heads (layer 0)."""
    _run("bf16", H=32, Hkv=2, hd=128, B=16, plens=[65536] * 4, qscale=0.5)
