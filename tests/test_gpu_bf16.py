"""GPU parity on the bf16 batch-1 tower at full size (prefix 4096, d 2048, 16 x 128 heads,
8 layers, MLP 8192, vocab 131072, block 16, gamma 0.8).

Logits within 2e-2 per-row relative error of the float64 oracle; decisions per step
from the oracle's state bit-exact except at exempt positions; the device-driven block
loop against the oracle's loop.
"""
import numpy as np
import pytest

from tests.gpu_common import (build_case, check_logits, conf_abs_err, conf_violations, decision_mismatches, gpu_step,
                              log, logits_rel_err)

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


@pytest.fixture(scope="module")
def b1():
    from synth import get_workload
    return build_case(get_workload("b1_p4096"))


@pytest.fixture(scope="module")
def b1_trace(b1):
    from oracle import oracle_generate
    w = b1.w
    return oracle_generate(b1.orc, w.n, w.B, b1.tau, w.gamma, b1.kv)


def test_step0_logits(b1, b1_trace):
    w = b1.w
    tok = np.full((w.n, w.B), w.V, dtype=np.int64)
    c = np.zeros((w.n, w.B), bool)
    g = gpu_step(b1, tok, c, w.gamma, want_logits=True)
    from oracle import oracle_step
    r = oracle_step(b1.orc, tok, c, b1.tau, w.gamma, b1.kv, keep_logits=True)
    err = logits_rel_err(g["z"].reshape(-1, w.V), r.z.reshape(-1, w.V))
    log(f"[b1] step0 logits rel err: max {err.max():.3e} mean {err.mean():.3e}; "
        f"conf abs err {conf_abs_err(g, r, c):.3e}")
    assert err.max() <= TOL_BF16
    check_logits(err, w.dtype, "b1 step 0")
    assert conf_violations(g, r, c, b1.tau, w.dtype, g["z"], r.z) == []
    bad = decision_mismatches(g, r, c, w.gamma)
    assert bad == [], bad


def test_teacher_forced_trace(b1, b1_trace):
    w = b1.w
    tok = np.full((w.n, w.B), w.V, dtype=np.int64)
    c = np.zeros((w.n, w.B), bool)
    all_bad = []
    for t, r in enumerate(b1_trace[3]):
        g = gpu_step(b1, tok, c, w.gamma)
        bad = decision_mismatches(g, r, c, w.gamma)
        log(f"[b1] step {t}: commits oracle {int(r.U.sum())} gpu {int(g['U'].sum())}, "
            f"conf abs err {conf_abs_err(g, r, c):.2e}, mismatches {len(bad)}")
        all_bad += [f"step {t}: {b}" for b in bad]
        all_bad += [f"step {t}: {b}" for b in conf_violations(g, r, c, b1.tau, w.dtype)]
        tok, c = r.tok, r.committed
    assert all_bad == [], all_bad


def test_generate_block(b1, b1_trace):
    w = b1.w
    torch = b1.torch
    tok_o, cs_o, steps_o, _ = b1_trace
    tok = torch.zeros((w.n, w.B), dtype=torch.int32, device="cuda")
    com = torch.zeros((w.n, w.B), dtype=torch.uint8, device="cuda")
    steps = torch.zeros(w.n, dtype=torch.int32, device="cuda")
    cstep = torch.zeros((w.n, w.B), dtype=torch.int8, device="cuda")
    b1.dev.generate_block(tok, com, b1.tau_d, w.gamma, steps=steps, commit_step=cstep)
    b1.dev.sync()
    tg, cg, sg = tok.cpu().numpy(), cstep.cpu().numpy(), steps.cpu().numpy()
    log(f"[b1] generate: steps gpu {sg} oracle {steps_o}; tokens equal {np.array_equal(tg, tok_o)}; "
        f"commit order equal {np.array_equal(cg, cs_o)}")
    assert com.cpu().numpy().all() and (sg <= w.B).all()
    assert np.array_equal(tg, tok_o) and np.array_equal(cg, cs_o) and np.array_equal(sg, steps_o)


@pytest.mark.parametrize("rule,k", [(0, 4), (1, 1)])
def test_generate_block_commit_rules(b1, rule, k):
    """The commit-rule variants at full size: the top 4 forced with the threshold, and the
    left-to-right mock-AR rule (16 steps, position p adopted at step p)."""
    from tests.test_gpu_batched import _check_generate
    _check_generate(b1, [0], b1.w.gamma, rule, k)
