"""GPU parity on batched towers: many sequences per call, ragged prefixes, GQA, B = 8/16/32.

Small towers (oracle on every sequence) exercise the multi-tile GEMM and LM-head paths
(M = n*B > 16, K split over workgroups, and the tiled kernel at M >= 128), ragged split-K
attention with empty and one-token prefixes, grouped-query heads and every block size.
The full-size batched workloads (ragged 32 x U{512..8192};
4 x 65536 GQA on the d 4096 tower; 64 x U{1024..4096} at B 8/16/32 and gamma 0.5/0.8/0.95)
run the whole batch on the GPU and check a fixed sample of sequences against the oracle:
sequences never interact (each has its own prefix, block and loop), so the oracle of a
sample is the oracle of those rows of the batch.  Bars: logits per-row relative error
(1e-4 fp32, 2e-2 bf16), decisions bit-exact outside the near-threshold / near-tie
exemptions, and the device-driven block loop equal to the oracle's loop.
"""
import numpy as np
import pytest

from tests.gpu_common import (build_case, check_logits, conf_abs_err, conf_violations, decision_mismatches, gpu_step,
                              log, logits_rel_err)

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _sample(plens, k):
    """Shortest prefix, longest prefix, then evenly spaced batch indices (deterministic)."""
    n = len(plens)
    pick = [int(np.argmin(plens)), int(np.argmax(plens))]
    for i in np.linspace(0, n - 1, k).astype(int):
        if len(pick) >= k:
            break
        if int(i) not in pick:
            pick.append(int(i))
    return sorted(pick[:k])


def _check_step0(case, sample):
    """Step 0 of the whole batch on the GPU; logits and decisions of `sample` vs the oracle."""
    from oracle import oracle_step
    w = case.w
    tok = np.full((w.n, w.B), w.V, dtype=np.int64)
    c = np.zeros((w.n, w.B), bool)
    g = gpu_step(case, tok, c, w.gamma, want_logits=True)
    r = oracle_step(case.orc, tok[sample], c[sample], case.tau[sample], w.gamma, case.kv, seqs=sample,
                    keep_logits=True)
    err = logits_rel_err(g["z"][sample].reshape(-1, w.V), r.z.reshape(-1, w.V))
    gs = {k: v[sample] for k, v in g.items() if k != "z"}
    log(f"[{w.name}] step0 sample {sample}: logits rel err max {err.max():.3e}; "
        f"conf abs err {conf_abs_err(gs, r, c[sample]):.2e}")
    assert err.max() <= TOL[w.dtype]
    check_logits(err, w.dtype, f"{w.name} step 0")
    assert conf_violations(gs, r, c[sample], case.tau[sample], w.dtype, g["z"][sample], r.z) == []
    bad = decision_mismatches(gs, r, c[sample], w.gamma)
    assert bad == [], bad


def _check_generate(case, sample, gamma, rule=0, min_adopt=1):
    """td_generate_block on the whole batch; the sample's tokens, commit steps, step counts."""
    from oracle import oracle_generate
    w = case.w
    torch = case.torch
    tok_o, cs_o, steps_o, _ = oracle_generate(case.orc, len(sample), w.B, case.tau[sample], gamma, case.kv,
                                              seqs=sample, keep_trace=False, rule=rule, min_adopt=min_adopt)
    tok = torch.zeros((w.n, w.B), dtype=torch.int32, device="cuda")
    com = torch.zeros((w.n, w.B), dtype=torch.uint8, device="cuda")
    steps = torch.zeros(w.n, dtype=torch.int32, device="cuda")
    cstep = torch.zeros((w.n, w.B), dtype=torch.int8, device="cuda")
    case.dev.set_commit_rule(rule, min_adopt)
    try:
        case.dev.generate_block(tok, com, case.tau_d, gamma, steps=steps, commit_step=cstep)
        case.dev.sync()
    finally:
        case.dev.set_commit_rule(0, 1)
    tg, cg, sg = tok.cpu().numpy(), cstep.cpu().numpy(), steps.cpu().numpy()
    log(f"[{w.name}] generate gamma {gamma} rule {rule} min_adopt {min_adopt}: steps gpu {sg[sample]} oracle "
        f"{steps_o}; batch steps min {sg.min()} max {sg.max()}")
    assert com.cpu().numpy().all() and (sg >= 1).all() and (sg <= w.B).all()
    assert np.array_equal(tg[sample], tok_o)
    assert np.array_equal(cg[sample], cs_o)
    assert np.array_equal(sg[sample], steps_o)


def _check_trace(case, sample, rule=0, min_adopt=1):
    """Teacher-forced steps: the sample follows the oracle's states; the other sequences of
    the batch are fully committed (they still run through the layers, never the LM head)."""
    from oracle import oracle_generate
    w = case.w
    _, _, _, trace = oracle_generate(case.orc, len(sample), w.B, case.tau[sample], w.gamma, case.kv, seqs=sample,
                                     rule=rule, min_adopt=min_adopt)
    tok = np.zeros((w.n, w.B), dtype=np.int64)
    c = np.ones((w.n, w.B), bool)
    tok[sample] = w.V
    c[sample] = False
    case.dev.set_commit_rule(rule, min_adopt)
    try:
        for t, r in enumerate(trace):
            g = gpu_step(case, tok, c, w.gamma)
            gs = {k: v[sample] for k, v in g.items()}
            bad = decision_mismatches(gs, r, c[sample], w.gamma, rule, min_adopt)
            log(f"[{w.name}] step {t} (rule {rule}, min_adopt {min_adopt}): commits oracle {int(r.U.sum())} gpu "
                f"{int(gs['U'].sum())}, conf err {conf_abs_err(gs, r, c[sample]):.2e}")
            assert bad == [], f"step {t}: {bad}"
            cbad = conf_violations(gs, r, c[sample], case.tau[sample], w.dtype)
            assert cbad == [], f"step {t}: {cbad}"
            others = np.setdiff1d(np.arange(w.n), sample)
            assert not g["U"][others].any(), "a committed sequence adopted a position"
            tok[sample], c[sample] = r.tok, r.committed
    finally:
        case.dev.set_commit_rule(0, 1)


# ---------------------------------------------------------------- small towers, every sequence checked
SMALL = {
    # M = 80: two 64-row GEMM tiles, the second partial; empty prefixes possible.
    "f32_n5_b16": dict(n=5, plen=("uniform", 0, 300), B=16, d=256, H=4, Hkv=2, hd=64, L=2, F=1024, V=4096,
                       dtype="f32"),
    # M = 96, R = G*B = 128 query rows per K/V head: the grouped-query attention path.
    "bf16_n3_b32_gqa": dict(n=3, plen=("uniform", 1, 700), B=32, d=256, H=8, Hkv=2, hd=64, L=2, F=1024, V=4096,
                            dtype="bf16"),
    # M = 72, head dim 128, block 8.
    "bf16_n9_b8": dict(n=9, plen=("uniform", 0, 100), B=8, d=256, H=4, Hkv=4, hd=128, L=2, F=512, V=4096,
                       dtype="bf16"),
    # M = 80, MLP down projection 512 x 4096: K split over two workgroups per column
    # group (fp32 partials summed in split order by a second kernel), two row tiles, the
    # second partial.
    "bf16_n5_b16_split": dict(n=5, plen=("uniform", 0, 300), B=16, d=512, H=4, Hkv=2, hd=128, L=2, F=4096,
                              V=4096, dtype="bf16"),
    # At most 16 rows: the LM head with the activations staged in LDS, all rows multiplied
    # and statistics written for the masked ones at their row-list position; M = 8 (rows
    # 8..15 padding) and two sequences in M = 16.
    "bf16_n1_b8_lds": dict(n=1, plen=("uniform", 1, 300), B=8, d=256, H=4, Hkv=4, hd=64, L=2, F=1024, V=4096,
                           dtype="bf16"),
    "bf16_n2_b8_lds": dict(n=2, plen=("uniform", 0, 300), B=8, d=512, H=4, Hkv=2, hd=128, L=2, F=2048, V=4096,
                           dtype="bf16"),
    # M = 144: the tiled many-row GEMM (128-row tiles, the second one partial) for every
    # projection and the LM head.
    "bf16_n9_b16_tiled": dict(n=9, plen=("uniform", 0, 200), B=16, d=256, H=4, Hkv=2, hd=64, L=2, F=1024,
                              V=4096, dtype="bf16"),
    # M = 48 (three row tiles, a four-tile group's last one empty), MLP 256 x 8192: four
    # column tiles per wave over eight waves; the down projection also K-split.
    "bf16_n3_b16_nt4": dict(n=3, plen=("uniform", 0, 200), B=16, d=256, H=4, Hkv=2, hd=64, L=2, F=8192,
                            V=4096, dtype="bf16"),
    # M = 400, MLP up projection 400 x 8192: 256 tiles of 128 rows, so 64-row tiles (the
    # last one partial, 16 rows); the down projection K-split over 16 workgroups.
    "bf16_n25_b16_tiled64": dict(n=25, plen=("uniform", 0, 100), B=16, d=256, H=4, Hkv=2, hd=64, L=2, F=8192,
                                 V=4096, dtype="bf16"),
}


@pytest.fixture(scope="module", params=sorted(SMALL))
def small(request):
    from synth import Workload
    kw = dict(SMALL[request.param])
    w = Workload(name=request.param, tower="small_" + request.param, weight_std=0.02, **kw)
    case = build_case(w)
    yield case
    case.dev.close()


def test_small_step0(small):
    _check_step0(small, list(range(small.w.n)))


def test_small_trace(small):
    _check_trace(small, list(range(small.w.n)))


def test_small_generate(small):
    _check_generate(small, list(range(small.w.n)), small.w.gamma)


# Commit-rule variants: the top k forced together with the threshold (k = 3 at the tower's
# gamma and at gamma > 1, exactly k per step) and the left-to-right mock-AR rule.
@pytest.mark.parametrize("rule,k,gamma", [(0, 3, None), (0, 3, 1.5), (1, 1, None)])
def test_small_generate_commit_rules(small, rule, k, gamma):
    _check_generate(small, list(range(small.w.n)), small.w.gamma if gamma is None else gamma, rule, k)


def test_small_trace_top3(small):
    _check_trace(small, list(range(small.w.n)), rule=0, min_adopt=3)


# ---------------------------------------------------------------- full-size batched workloads
@pytest.fixture(scope="module")
def ragged32():
    from synth import get_workload
    case = build_case(get_workload("ragged32"))
    yield case
    case.dev.close()


def test_ragged32_step0(ragged32):
    _check_step0(ragged32, _sample(ragged32.plens, 3))


def test_ragged32_generate(ragged32):
    _check_generate(ragged32, _sample(ragged32.plens, 4), ragged32.w.gamma)


@pytest.fixture(scope="module")
def gqa_long():
    from synth import get_workload
    case = build_case(get_workload("gqa_long"))
    yield case
    case.dev.close()


def test_gqa_long_step0(gqa_long):
    _check_step0(gqa_long, [0, 3])


def test_gqa_long_generate(gqa_long):
    _check_generate(gqa_long, [1], gqa_long.w.gamma)


@pytest.fixture(scope="module", params=["sweep64_b8", "sweep64_b16", "sweep64_b32"])
def sweep(request):
    from synth import get_workload
    case = build_case(get_workload(request.param))
    yield case
    case.dev.close()


def test_sweep_step0(sweep):
    _check_step0(sweep, _sample(sweep.plens, 2))


@pytest.mark.parametrize("gamma", [0.5, 0.8, 0.95])
def test_sweep_generate(sweep, gamma):
    _check_generate(sweep, _sample(sweep.plens, 2), gamma)
