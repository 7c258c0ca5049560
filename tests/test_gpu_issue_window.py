"""GPU: td_generate_block with an issue window (td_set_issue_window) gives the results of
the whole loop issued at once; the window only leaves out launches that would return on
the device's loop-exit flag.

Compared bit for bit with window 0 (itself checked against the oracle's block loop in the
tiny, batched and full-size tests) and, on the tiny tower, with the oracle's loop.
"""
import time

import numpy as np
import pytest

from tests.gpu_common import build_case, log

pytestmark = pytest.mark.gpu


def _run(case, gamma, window):
    torch, w = case.torch, case.w
    case.dev.set_issue_window(window)
    try:
        tok = torch.zeros((w.n, w.B), dtype=torch.int32, device="cuda")
        com = torch.zeros((w.n, w.B), dtype=torch.uint8, device="cuda")
        steps = torch.zeros(w.n, dtype=torch.int32, device="cuda")
        cstep = torch.zeros((w.n, w.B), dtype=torch.int8, device="cuda")
        case.dev.generate_block(tok, com, case.tau_d, gamma, steps=steps, commit_step=cstep)
        case.dev.sync()
    finally:
        case.dev.set_issue_window(0)
    return tuple(x.cpu().numpy() for x in (tok, com, steps, cstep))


def _same(ref, got):
    return all(np.array_equal(a, b) for a, b in zip(ref, got))


@pytest.fixture(scope="module")
def tiny():
    from synth import get_workload
    return build_case(get_workload("tiny_fp32"))


@pytest.fixture(scope="module")
def batch():
    from synth import Workload
    # Nine sequences finishing at different steps (block 8, bf16).
    w = Workload(name="window_n9_b8", tower="small_window_n9_b8", n=9, plen=("uniform", 0, 100), B=8, d=256, H=4,
                 Hkv=4, hd=128, L=2, F=512, V=4096, dtype="bf16")
    case = build_case(w)
    yield case
    case.dev.close()


# gamma 0 adopts everything in the first step (the loop stops after one step); 1.5 adopts
# one position per step (every step is needed).
@pytest.mark.parametrize("gamma", [0.8, 0.95, 1.5, 0.0])
def test_tiny_windows_match_whole_loop(tiny, gamma):
    ref = _run(tiny, gamma, 0)
    log(f"[window] tiny gamma {gamma}: {int(ref[2][0])} steps")
    for win in (1, 2, 3, tiny.w.B):
        assert _same(ref, _run(tiny, gamma, win)), f"window {win}"


def test_tiny_window_matches_oracle(tiny):
    from oracle import oracle_generate
    w = tiny.w
    tok_o, cs_o, steps_o, _ = oracle_generate(tiny.orc, w.n, w.B, tiny.tau, w.gamma, tiny.kv)
    tok, com, steps, cstep = _run(tiny, w.gamma, 2)
    assert com.all()
    assert np.array_equal(tok, tok_o)
    assert np.array_equal(cstep, cs_o)
    assert np.array_equal(steps, steps_o)


@pytest.mark.parametrize("gamma", [None, 1.5])
def test_batch_windows_match_whole_loop(batch, gamma):
    g = batch.w.gamma if gamma is None else gamma
    ref = _run(batch, g, 0)
    log(f"[window] batch gamma {g}: steps {ref[2].tolist()}")
    for win in (1, 2):
        assert _same(ref, _run(batch, g, win)), f"window {win}"


def test_window_must_not_be_negative(tiny):
    from block_diffusion_lm_step_amd import TD_EINVAL, TdError
    with pytest.raises(TdError) as ei:
        tiny.dev.set_issue_window(-1)
    assert ei.value.status == TD_EINVAL


def test_window_falls_back_when_the_device_reports_nothing(tiny):
    """The stream is still busy with earlier work (a bounded spin kernel of about 3 s,
    enqueued first), so no progress arrives: the first wait gives up after a second, the
    call enqueues the remaining steps at once and returns, and the results are those of
    the whole loop."""
    torch, w = tiny.torch, tiny.w
    ref = _run(tiny, w.gamma, 0)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 20_000_000
    start.record()
    torch.cuda._sleep(n)
    stop.record()
    stop.synchronize()
    per_s = n / (start.elapsed_time(stop) * 1e-3)   # spin-kernel cycles per second
    tok = torch.zeros((w.n, w.B), dtype=torch.int32, device="cuda")
    com = torch.zeros((w.n, w.B), dtype=torch.uint8, device="cuda")
    steps = torch.zeros(w.n, dtype=torch.int32, device="cuda")
    cstep = torch.zeros((w.n, w.B), dtype=torch.int8, device="cuda")
    tiny.dev.set_issue_window(2)
    try:
        torch.cuda._sleep(int(3.0 * per_s))
        t0 = time.perf_counter()
        tiny.dev.generate_block(tok, com, tiny.tau_d, w.gamma, steps=steps, commit_step=cstep)
        returned = time.perf_counter() - t0
        tiny.dev.sync()
    finally:
        tiny.dev.set_issue_window(0)
    log(f"[window] busy stream: generate_block returned after {returned:.2f} s")
    assert 0.9 <= returned < 2.5
    assert _same(ref, tuple(x.cpu().numpy() for x in (tok, com, steps, cstep)))
