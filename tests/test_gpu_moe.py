"""GPU parity of the mixture-of-experts denoiser (td_set_moe) against the float64 oracle.

Small towers cover fp32 and bf16 storage, expert counts that are not a multiple of 32
(padded router), 256 experts, top_k up to 8 and top_k = E, no shared expert, several
16-row tiles per expert (M = 144: the tiled router GEMM and separate routing and bucket
kernels; the others route and bucket in one workgroup) and a single row per expert; the full-size tower is the
batch-1 d 2048 tower with 128 experts, 6 routed + 2 shared of width 1024.

Bars: logits per-row relative error (1e-4 fp32, 2e-2 bf16), decisions bit-exact outside
the near-threshold / near-tie exemptions, the device block loop equal to the oracle's,
and the routing itself: the number of distinct experts the device routed rows to in
every layer of every step (td_moe_stats) equals the oracle's.

Routing is a float decision taken on fp32 router scores.  The device's scores differ from
the float64 ones by the bf16 high/remainder split of the normed input (relative 2^-17
per element) summed over d terms: about 2^-17 * 0.02 * sqrt(d) ~ 7e-6 at d = 2048 for
these weights.  A teacher-forced step in which some row's k-th and (k+1)-th oracle
scores are closer than ROUTE_MARGIN (several times that) is a near-tie: its routing, and
so its logits and decisions, may legitimately differ; such steps are logged and skipped,
and at least half of a trace's steps must be checked.
"""
import numpy as np
import pytest

from tests.gpu_common import (build_case, check_logits, conf_abs_err, conf_violations, decision_mismatches, gpu_step,
                              log, logits_rel_err)

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
ROUTE_MARGIN = 3e-5


def _route_info(case, tok, seqs, per_seq=False, committed=None):
    """Oracle routing of token blocks tok [S][B]: distinct active experts (routed with a
    row, plus shared) summed over the layers, and the smallest top-k margin (of each
    sequence with per_seq).  With several sequences the device routes no row of a
    sequence whose block is adopted (`committed` all true), so those rows count for no
    expert."""
    cap = {}
    case.orc.hidden(tok, case.kv, seqs, capture=cap)
    E, k, S, _ = case.w.moe
    live = np.ones(tok.shape[0], bool)
    if committed is not None and tok.shape[0] > 1:
        live = ~committed.all(axis=1)
    active, margin = 0, np.full(tok.shape[0], np.inf)
    for ex, sc in zip(cap["experts"], cap["scores"]):
        active += len(np.unique(ex[live])) + S
        if k < E:
            s32 = np.sort(sc.astype(np.float32).astype(np.float64), axis=2)[:, :, ::-1]
            margin = np.minimum(margin, (s32[:, :, k - 1] - s32[:, :, k]).min(axis=1))
    return active, (margin if per_seq else float(margin.min()))


# Seeds: ones whose oracle block loops have few routing near-ties (checked on the CPU).
SMALL = {
    # fp32 storage, 8 experts top-2 + 1 shared, M = 32.
    "f32_e8_k2_s1": dict(n=2, plen=("uniform", 0, 300), B=16, d=256, H=4, Hkv=2, hd=64, L=2, F=1024, V=4096,
                         dtype="f32", moe=(8, 2, 1, 128), seed=1),
    # 40 experts (router padded to 64 columns), top-6 + 2 shared, M = 48.
    "bf16_e40_k6_s2": dict(n=3, plen=("uniform", 0, 300), B=16, d=512, H=4, Hkv=4, hd=128, L=2, F=2048, V=4096,
                           dtype="bf16", moe=(40, 6, 2, 256), seed=1),
    # M = 144: the tiled router GEMM, several 16-row tiles per expert.
    "bf16_e16_k4_s1_n9": dict(n=9, plen=("uniform", 0, 200), B=16, d=256, H=4, Hkv=2, hd=64, L=2, F=1024, V=4096,
                              dtype="bf16", moe=(16, 4, 1, 128), seed=3),
    # top_k = 8 (the maximum), no shared expert, block 8.
    "bf16_e32_k8_s0_b8": dict(n=1, plen=("uniform", 1, 300), B=8, d=256, H=4, Hkv=4, hd=64, L=2, F=1024, V=4096,
                              dtype="bf16", moe=(32, 8, 0, 64)),
    # 256 experts (the maximum: four router scores per lane), top 3.
    "bf16_e256_k3_s0": dict(n=2, plen=("uniform", 0, 200), B=16, d=256, H=4, Hkv=4, hd=64, L=2, F=1024, V=4096,
                            dtype="bf16", moe=(256, 3, 0, 64), seed=2),
    # top_k = E: every expert chosen, routing decides only the gates.
    "f32_e4_k4_s1": dict(n=2, plen=("uniform", 0, 200), B=8, d=256, H=4, Hkv=2, hd=64, L=2, F=1024, V=4096,
                         dtype="f32", moe=(4, 4, 1, 64)),
}


@pytest.fixture(scope="module", params=sorted(SMALL))
def small(request):
    from synth import Workload
    kw = dict(SMALL[request.param])
    w = Workload(name="moe_" + request.param, tower="moe_" + request.param, **kw)
    case = build_case(w)
    yield case
    case.dev.close()


def _check_trace(case, steps=None):
    """Teacher-forced steps from the oracle's states (the oracle's block loop, one step at a
    time): logits, decisions and per-step routing."""
    from oracle import oracle_step
    w = case.w
    seqs = list(range(w.n))
    tok = np.full((w.n, w.B), w.V, dtype=np.int64)
    c = np.zeros((w.n, w.B), bool)
    case.dev.moe_stats()   # reset
    t = checked = 0
    while not c.all() and (steps is None or t < steps):
        active, margin = _route_info(case, tok, seqs, committed=c)
        g = gpu_step(case, tok, c, w.gamma, want_logits=True)
        launches, act_gpu = case.dev.moe_stats()
        masked = ~c
        r = oracle_step(case.orc, tok, c, case.tau, w.gamma, case.kv, seqs=seqs, keep_logits=True)
        err = logits_rel_err(g["z"][masked], r.z[masked])
        bad = decision_mismatches(g, r, c, w.gamma)
        log(f"[{w.name}] step {t}: logits rel err {err.max():.3e}, conf err {conf_abs_err(g, r, c):.2e}, "
            f"active experts gpu {act_gpu} oracle {active} over {launches} layers, route margin {margin:.2e}")
        assert launches == w.L
        if margin > ROUTE_MARGIN:
            assert act_gpu == active
            assert err.max() <= TOL[w.dtype]
            check_logits(err, w.dtype, f"{w.name} step {t}")
            cbad = conf_violations(g, r, c, case.tau, w.dtype, g["z"], r.z)
            assert cbad == [], f"step {t}: {cbad}"
            assert bad == [], f"step {t}: {bad}"
            checked += 1
        else:
            log(f"[{w.name}] step {t}: near-tie in the oracle's routing, step not compared")
        tok, c = r.tok, r.committed
        t += 1
    assert 2 * checked >= t, f"only {checked} of {t} steps free of routing near-ties"


def test_small_moe_trace(small):
    _check_trace(small)


def test_small_moe_generate(small):
    """The device block loop against the oracle's.  Sequences never interact, so a
    sequence whose oracle loop meets a routing near-tie is left out of the comparison (at
    least half must remain)."""
    from oracle import oracle_generate
    case = small
    w = case.w
    torch = case.torch
    tok_o, cs_o, steps_o, trace = oracle_generate(case.orc, w.n, w.B, case.tau, w.gamma, case.kv)
    margin = np.full(w.n, np.inf)
    state = np.full((w.n, w.B), w.V, dtype=np.int64)
    for r in trace:
        margin = np.minimum(margin, _route_info(case, state, list(range(w.n)), per_seq=True)[1])
        state = r.tok
    keep = margin > ROUTE_MARGIN
    assert 2 * keep.sum() >= w.n, f"routing near-ties in {int((~keep).sum())} of {w.n} sequences"
    tok = torch.zeros((w.n, w.B), dtype=torch.int32, device="cuda")
    com = torch.zeros((w.n, w.B), dtype=torch.uint8, device="cuda")
    steps = torch.zeros(w.n, dtype=torch.int32, device="cuda")
    cstep = torch.zeros((w.n, w.B), dtype=torch.int8, device="cuda")
    case.dev.moe_stats()
    case.dev.generate_block(tok, com, case.tau_d, w.gamma, steps=steps, commit_step=cstep)
    case.dev.sync()
    launches, _ = case.dev.moe_stats()
    sg = steps.cpu().numpy()
    log(f"[{w.name}] generate: steps gpu {sg} oracle {steps_o}; expert layers run {launches}; compared "
        f"sequences {np.nonzero(keep)[0].tolist()}")
    assert np.array_equal(tok.cpu().numpy()[keep], tok_o[keep])
    assert np.array_equal(cstep.cpu().numpy()[keep], cs_o[keep])
    assert np.array_equal(sg[keep], steps_o[keep])
    assert launches == w.L * int(sg.max())   # the layers of finished steps exit on the device flag


def test_moe_determinism(small):
    """Rows land in their expert's segment in an order set by LDS atomics, but every output
    row is computed from its own input row only and the gated sum is in slot order: two
    runs give bit-identical logits and decisions."""
    w = small.w
    tok = np.full((w.n, w.B), w.V, dtype=np.int64)
    c = np.zeros((w.n, w.B), bool)
    g1 = gpu_step(small, tok, c, w.gamma, want_logits=True)
    g2 = gpu_step(small, tok, c, w.gamma, want_logits=True)
    assert np.array_equal(g1["z"], g2["z"], equal_nan=True)
    assert np.array_equal(g1["tok"], g2["tok"]) and np.array_equal(g1["conf"], g2["conf"], equal_nan=True)


def test_moe_rejects_bad_configs(small):
    from block_diffusion_lm_step_amd import TdError
    w = small.w
    E, k, S, de = w.moe
    for bad in (dict(n_experts=0, top_k=1, n_shared=0, d_expert=64), dict(n_experts=E, top_k=E + 1, n_shared=0,
                d_expert=64), dict(n_experts=E, top_k=9, n_shared=0, d_expert=64),
                dict(n_experts=E, top_k=k, n_shared=5, d_expert=64), dict(n_experts=E, top_k=k, n_shared=0, d_expert=96)):
        with pytest.raises(TdError):
            small.dev.set_moe(bad, dict(router=None, w1=None, w2=None))
    # the ctx keeps its experts after a rejected call
    from tests.gpu_common import gpu_step as _g
    tok = np.full((w.n, w.B), w.V, dtype=np.int64)
    _g(small, tok, np.zeros((w.n, w.B), bool), w.gamma)


def test_moe_full_size_first_steps():
    """The batch-1 d 2048 tower with 128 experts (6 + 2 shared, width 1024): the first two
    teacher-forced steps against the oracle."""
    from synth import get_workload
    case = build_case(get_workload("moe_b1_p4096"))
    try:
        _check_trace(case, steps=2)
    finally:
        case.dev.close()


def test_moe_errors_without_experts():
    """A tower created without dense MLP weights cannot step until td_set_moe; td_moe_stats
    needs a mixture of experts."""
    import torch
    from block_diffusion_lm_step_amd import Denoiser, TdError
    from synth import Workload, draw_prefix_lengths, draw_tower
    from synth.device import prefix_to_device, tower_config, tower_to_device
    w = Workload(name="moe_noexp", tower="moe_noexp", n=1, plen=("fixed", 40), B=8, d=256, H=4, Hkv=4, hd=64, L=1,
                 F=1024, V=4096, dtype="bf16", moe=(8, 2, 0, 64))
    dW = tower_to_device(draw_tower(w))
    assert dW["w1"] is None and dW["w2"] is None
    offsets, ks, vs = prefix_to_device(w, draw_prefix_lengths(w))
    dev = Denoiser(tower_config(w, max_batch=1, max_prefix_tokens=offsets[-1]), dW)
    try:
        dev.set_prefix(offsets, ks, vs)
        tok = torch.full((1, w.B), w.V, dtype=torch.int32, device="cuda")
        com = torch.zeros((1, w.B), dtype=torch.uint8, device="cuda")
        with pytest.raises(TdError, match="no MLP"):
            dev.denoise_step(tok, com, None, w.gamma)
        with pytest.raises(TdError, match="no MLP"):
            dev.generate_block(tok, com, None, w.gamma)
        with pytest.raises(TdError, match="mixture of experts"):
            dev.moe_stats()
        dev.sync()
    finally:
        dev.close()
