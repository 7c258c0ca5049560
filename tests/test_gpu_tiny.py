"""GPU parity on the tiny fp32 tower (d 256, 4 heads x 64, 2 layers, vocab 4096, prefix 128).

Every call goes through the C ABI (libtd) via the thin binding.  Tolerance: logits 1e-4
relative per row; decisions bit-exact with the near-threshold / near-tie exemptions.
"""
import numpy as np
import pytest

from tests.gpu_common import (EXEMPT, build_case, check_logits, conf_abs_err, conf_violations, decision_mismatches,
                              gpu_step, log, logits_rel_err)

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4


@pytest.fixture(scope="module")
def tiny():
    from synth import get_workload
    return build_case(get_workload("tiny_fp32"))


def test_step_from_all_mask(tiny):
    from oracle import oracle_step
    w = tiny.w
    tok = np.full((w.n, w.B), w.V, dtype=np.int64)
    c = np.zeros((w.n, w.B), bool)
    g = gpu_step(tiny, tok, c, w.gamma, want_logits=True)
    r = oracle_step(tiny.orc, tok, c, tiny.tau, w.gamma, tiny.kv, keep_logits=True)
    err = logits_rel_err(g["z"].reshape(-1, w.V), r.z.reshape(-1, w.V))
    log(f"[tiny] step0 logits rel err max {err.max():.3e}; conf abs err {conf_abs_err(g, r, c):.3e}")
    assert err.max() <= TOL_F32
    check_logits(err, w.dtype, "tiny step 0")
    assert conf_violations(g, r, c, tiny.tau, w.dtype, g["z"], r.z) == []
    assert decision_mismatches(g, r, c, w.gamma) == []
    assert np.array_equal(g["committed"], r.committed) or decision_mismatches(g, r, c, w.gamma) == []


def test_teacher_forced_trace(tiny):
    from oracle import oracle_generate
    w = tiny.w
    _, _, _, trace = oracle_generate(tiny.orc, w.n, w.B, tiny.tau, w.gamma, tiny.kv)
    tok = np.full((w.n, w.B), w.V, dtype=np.int64)
    c = np.zeros((w.n, w.B), bool)
    for t, r in enumerate(trace):
        g = gpu_step(tiny, tok, c, w.gamma)
        bad = decision_mismatches(g, r, c, w.gamma)
        log(f"[tiny] step {t}: commits oracle {r.U.sum()} gpu {g['U'].sum()}, conf err {conf_abs_err(g, r, c):.2e}")
        assert bad == [], bad
        assert conf_violations(g, r, c, tiny.tau, w.dtype) == []
        tok, c = r.tok, r.committed


def test_generate_block_matches_oracle(tiny):
    from oracle import oracle_generate
    w = tiny.w
    torch = tiny.torch
    tok_o, cs_o, steps_o, _ = oracle_generate(tiny.orc, w.n, w.B, tiny.tau, w.gamma, tiny.kv)
    tok = torch.zeros((w.n, w.B), dtype=torch.int32, device="cuda")
    com = torch.zeros((w.n, w.B), dtype=torch.uint8, device="cuda")
    steps = torch.zeros(w.n, dtype=torch.int32, device="cuda")
    cstep = torch.zeros((w.n, w.B), dtype=torch.int8, device="cuda")
    tiny.dev.generate_block(tok, com, tiny.tau_d, w.gamma, steps=steps, commit_step=cstep)
    tiny.dev.sync()
    log(f"[tiny] generate: steps gpu {steps.cpu().numpy()} oracle {steps_o}")
    assert com.cpu().numpy().all()
    assert np.array_equal(tok.cpu().numpy(), tok_o)
    assert np.array_equal(cstep.cpu().numpy(), cs_o)
    assert np.array_equal(steps.cpu().numpy(), steps_o)


@pytest.mark.parametrize("gamma", [0.0, 1.5])
def test_gamma_closed_forms(tiny, gamma):
    w = tiny.w
    torch = tiny.torch
    tok = torch.zeros((w.n, w.B), dtype=torch.int32, device="cuda")
    com = torch.zeros((w.n, w.B), dtype=torch.uint8, device="cuda")
    steps = torch.zeros(w.n, dtype=torch.int32, device="cuda")
    cstep = torch.zeros((w.n, w.B), dtype=torch.int8, device="cuda")
    tiny.dev.generate_block(tok, com, tiny.tau_d, gamma, steps=steps, commit_step=cstep)
    tiny.dev.sync()
    cs = cstep.cpu().numpy()
    if gamma == 0.0:
        assert (steps.cpu().numpy() == 1).all() and (cs == 0).all()
        # tokens equal the argmax of one forward from the all-[MASK] block
        g = gpu_step(tiny, np.full((w.n, w.B), w.V), np.zeros((w.n, w.B), bool), 0.0)
        assert np.array_equal(tok.cpu().numpy(), g["arg"])
    else:
        assert (steps.cpu().numpy() == w.B).all()
        for s in range(w.n):
            assert sorted(cs[s].tolist()) == list(range(w.B))


def test_determinism(tiny):
    w = tiny.w
    torch = tiny.torch
    outs = []
    for _ in range(2):
        tok = torch.zeros((w.n, w.B), dtype=torch.int32, device="cuda")
        com = torch.zeros((w.n, w.B), dtype=torch.uint8, device="cuda")
        cstep = torch.zeros((w.n, w.B), dtype=torch.int8, device="cuda")
        tiny.dev.generate_block(tok, com, tiny.tau_d, w.gamma, commit_step=cstep)
        g = gpu_step(tiny, np.full((w.n, w.B), w.V), np.zeros((w.n, w.B), bool), w.gamma, want_logits=True)
        outs.append((tok.cpu().numpy(), cstep.cpu().numpy(), g["conf"], g["z"]))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b, equal_nan=True)


def test_invalid_state_is_reported_not_faulted(tiny):
    from block_diffusion_lm_step_amd import TD_EDEVICE, TdError
    w = tiny.w
    tok = np.full((w.n, w.B), w.V, dtype=np.int64)
    c = np.zeros((w.n, w.B), bool)
    c[0, 3] = True            # committed but still [MASK]
    with pytest.raises(TdError) as ei:
        gpu_step(tiny, tok, c, w.gamma)
    assert ei.value.status == TD_EDEVICE
    tok[0, 5] = w.V + 7       # out-of-range id
    with pytest.raises(TdError):
        gpu_step(tiny, tok, np.zeros((w.n, w.B), bool), w.gamma)
    # the ctx stays usable afterwards
    g = gpu_step(tiny, np.full((w.n, w.B), w.V), np.zeros((w.n, w.B), bool), w.gamma)
    assert g["U"].any()
