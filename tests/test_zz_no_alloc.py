"""GPU test of the allocation-free step (td_denoise_step_noalloc) through the C ABI.

The variant must give exactly what td_denoise_step gives (same kernels, partial results
in the library's file-scope device array instead of the ctx's buffers), on two calls in
a row -- the second on a smaller bound batch, so it runs over what the first left in the
array -- must not change the device's free memory, and must refuse a bound batch whose
step scratch exceeds the array, leaving the ctx usable.
"""
import numpy as np
import pytest

from tests.gpu_common import build_case, log

pytestmark = pytest.mark.gpu


def _step(case, variant, tok, c, gamma, n):
    torch = case.torch
    w = case.w
    t_tok = torch.from_numpy(tok[:n].astype(np.int32)).cuda()
    t_c = torch.from_numpy(c[:n].astype(np.uint8)).cuda()
    newly = torch.zeros_like(t_c)
    conf = torch.full((n, w.B), float("nan"), dtype=torch.float32, device="cuda")
    arg = torch.full((n, w.B), -1, dtype=torch.int32, device="cuda")
    logits = torch.full((n, w.B, w.V), float("nan"), dtype=torch.float32, device="cuda")
    fn = case.dev.denoise_step_noalloc if variant else case.dev.denoise_step
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    fn(t_tok, t_c, case.tau_d[:n], gamma, newly=newly, conf=conf, argmax=arg, logits=logits)
    case.dev.sync()
    free1 = torch.cuda.mem_get_info()[0]
    return dict(tok=t_tok.cpu().numpy(), c=t_c.cpu().numpy(), newly=newly.cpu().numpy(), conf=conf.cpu().numpy(),
                arg=arg.cpu().numpy(), z=logits.cpu().numpy(), free_delta=free0 - free1)


def _same(a, b):
    for k in ("tok", "c", "newly", "conf", "arg", "z"):
        assert np.array_equal(a[k], b[k], equal_nan=True), k


@pytest.fixture(scope="module")
def case():
    from synth import Workload
    # 5 sequences, ragged prefixes (empty ones too), grouped-query heads, M = 80 rows: the
    # few-row LM head over the row list, K split in the MLP down projection.
    w = Workload(name="noalloc_n5", tower="noalloc_n5", n=5, plen=("uniform", 0, 400), B=16, d=512, H=8, Hkv=2, hd=64,
                 L=2, F=4096, V=8192, dtype="bf16")
    c = build_case(w)
    yield c
    c.dev.close()


def test_noalloc_step_equals_the_step_twice(case):
    from synth.device import prefix_to_device
    w = case.w
    rng = np.random.default_rng(7)
    c = rng.random((w.n, w.B)) < 0.3
    tok = np.where(c, rng.integers(0, w.V, (w.n, w.B)), w.V)
    ref = _step(case, False, tok, c, w.gamma, w.n)
    got = _step(case, True, tok, c, w.gamma, w.n)
    log(f"[noalloc] call 1: {int(got['newly'].sum())} adopted, free-memory change {got['free_delta']} B")
    _same(ref, got)
    assert got["free_delta"] == 0
    # Second call on a smaller bound batch: the first three sequences only.
    n2 = 3
    offsets, ks, vs = prefix_to_device(w, case.plens[:n2])
    case.dev.set_prefix(offsets, ks, vs)
    try:
        got2 = _step(case, True, tok, c, 0.5, n2)
        ref2 = _step(case, False, tok, c, 0.5, n2)
        log(f"[noalloc] call 2 (batch {n2}): {int(got2['newly'].sum())} adopted")
        _same(ref2, got2)
        assert got2["free_delta"] == 0
    finally:
        offsets, ks, vs = prefix_to_device(w, case.plens)
        case.dev.set_prefix(offsets, ks, vs)


def test_noalloc_rejects_a_batch_beyond_the_array():
    """2048 sequences of 32 positions: the attention partial states and vocabulary
    statistics of one step need more than the array holds."""
    import torch

    from block_diffusion_lm_step_amd import TD_EINVAL, Denoiser, TdError
    from synth import Workload, draw_tower
    from synth.device import tower_config, tower_to_device
    w = Workload(name="noalloc_big", tower="noalloc_big", n=2048, plen=("fixed", 0), B=32, d=256, H=4, Hkv=4, hd=64,
                 L=1, F=1024, V=4096, dtype="bf16")
    dev = Denoiser(tower_config(w, max_batch=w.n, max_prefix_tokens=1), tower_to_device(draw_tower(w)))
    try:
        dev.set_prefix([0] * (w.n + 1), [torch.zeros(1, device="cuda")], [torch.zeros(1, device="cuda")])
        tok = torch.full((w.n, w.B), w.V, dtype=torch.int32, device="cuda")
        com = torch.zeros((w.n, w.B), dtype=torch.uint8, device="cuda")
        with pytest.raises(TdError) as ei:
            dev.denoise_step_noalloc(tok, com, None, 0.8)
        assert ei.value.status == TD_EINVAL and "scratch" in str(ei.value)
        log(f"[noalloc] refused: {ei.value}")
        dev.denoise_step(tok, com, None, 0.8)   # the ctx stays usable
        dev.sync()
        assert com.cpu().numpy().any()
    finally:
        dev.close()
