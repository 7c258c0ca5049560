"""The C-ABI library on the CPU: it loads, exports every symbol include/td.h declares, and
rejects bad arguments on the host before any HIP call (no compute without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "td.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(td_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def td():
    import block_diffusion_lm_step_amd as td
    return td


def test_every_declared_symbol_is_exported(td):
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(td.lib, n), n
    assert set(names) == set(td.EXPORTED)


def test_version(td):
    assert td.lib.td_version().startswith(b"td ")


def _cfg(td, **kw):
    base = dict(n_layers=2, d_model=256, n_heads=4, n_kv_heads=4, head_dim=64, d_ff=1024, vocab=4096, block_size=16,
                max_batch=1, max_prefix_tokens=128, dtype=td.TD_F32, rms_eps=1e-6)
    base.update(kw)
    return td.TdConfig(*[base[f] for f, _ in td.TdConfig._fields_])


@pytest.mark.parametrize("bad", [dict(head_dim=96), dict(block_size=12), dict(n_heads=6, n_kv_heads=4),
                                 dict(d_model=100), dict(vocab=1000), dict(dtype=7), dict(max_batch=0),
                                 dict(rms_eps=float("nan")), dict(n_layers=0), dict(max_prefix_tokens=-1)])
def test_create_rejects_bad_config(td, bad):
    ctx = ctypes.c_void_p()
    w = td.TdWeights()
    st = td.lib.td_create(ctypes.byref(_cfg(td, **bad)), ctypes.byref(w), None, ctypes.byref(ctx))
    assert st == td.TD_EINVAL
    assert ctx.value is None
    assert td.lib.td_last_error(None)


def test_create_rejects_null_weights(td):
    ctx = ctypes.c_void_p()
    assert td.lib.td_create(ctypes.byref(_cfg(td)), None, None, ctypes.byref(ctx)) == td.TD_EINVAL
    w = td.TdWeights()   # all NULL
    assert td.lib.td_create(ctypes.byref(_cfg(td)), ctypes.byref(w), None, ctypes.byref(ctx)) == td.TD_EINVAL
    assert b"NULL" in td.lib.td_last_error(None)


def test_create_without_device_reports_device_error(td):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; this checks the GPU-less failure path")
    fake = (ctypes.c_void_p * 2)(16, 16)
    w = td.TdWeights(16, 16, fake, fake, fake, fake, fake, fake, fake, fake, 16, 16)
    ctx = ctypes.c_void_p()
    st = td.lib.td_create(ctypes.byref(_cfg(td)), ctypes.byref(w), None, ctypes.byref(ctx))
    assert st == td.TD_EDEVICE
    assert ctx.value is None
    assert b"device" in td.lib.td_last_error(None)


def test_null_ctx_calls_are_rejected(td):
    assert td.lib.td_set_prefix(None, 1, None, None, None) == td.TD_EINVAL
    assert td.lib.td_denoise_step(None, None, None, None, 0.8, None, None, None, None) == td.TD_EINVAL
    assert td.lib.td_generate_block(None, None, None, None, 0.8, None, None) == td.TD_EINVAL
    assert td.lib.td_debug_attention(None, 0, None, None) == td.TD_EINVAL
    assert td.lib.td_sync(None) == td.TD_EINVAL
    assert td.lib.td_profile_begin(None, 1) == td.TD_EINVAL
    assert td.lib.td_profile_layer(None, 0) == td.TD_EINVAL
    assert td.lib.td_profile_end(None, None, None, 0) == -1
    assert td.lib.td_kernels_per_step(None) == -1
    assert td.lib.td_set_commit_rule(None, 0, 1) == td.TD_EINVAL
    assert td.lib.td_set_issue_window(None, 2) == td.TD_EINVAL
    assert td.lib.td_bind_cache(None, 1, None, None, None, None) == td.TD_EINVAL
    assert td.lib.td_set_context_tower(None, None) == td.TD_EINVAL
    assert td.lib.td_append_block(None, None) == td.TD_EINVAL
    assert td.lib.td_ar_step(None, None) == td.TD_EINVAL
    assert td.lib.td_set_moe(None, None, None) == td.TD_EINVAL
    n, act = ctypes.c_int64(0), ctypes.c_int64(0)
    assert td.lib.td_moe_stats(None, ctypes.byref(n), ctypes.byref(act)) == td.TD_EINVAL
    td.lib.td_destroy(None)


def test_bench_refuses_several_gpus():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
