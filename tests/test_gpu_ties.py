"""Exact ties on the GPU: an all-zero LM head.

Every logit is then exactly 0 for every position, so each masked position's confidence is
1/V exactly (V equal terms exp(0) = 1; integer sums are exact in fp32 below 2^24, and 1/V
is a power of two for these vocabularies) and its prediction is vocabulary id 0, the
lowest id of the maximum (PredNext "人工知能は拡散言語モデルの夢を見るか？", section
拡散言語モデルで推論するには, step 3, with the single-position fallback: lowest position
on ties).  With gamma = 0.5 > 1/V no position clears the threshold, so each step adopts
exactly the lowest masked position: position p at step p, B steps, all tokens 0.

These exercise the tie breaks that random weights never reach: the lowest vocabulary id
across lanes, waves and workgroups of the LM-head kernels and in the merge of the column
groups, and the lowest position in the commit.  Bit-exact, no exemption.  Cases: the fp32
tiny tower, and d 256 bf16 towers with vocabulary 131072 on each LM-head kernel (16 rows
staged in LDS, 48 rows over the row list, 144 rows in 128 x 128 tiles with the two-launch
merge and commit).
"""
import numpy as np
import pytest

from tests.gpu_common import build_case, gpu_step, log

pytestmark = pytest.mark.gpu

GAMMA = 0.5
_BIGV = dict(plen=("uniform", 0, 300), B=16, d=256, H=4, Hkv=2, hd=64, L=2, F=1024, V=131072, dtype="bf16")
CASES = {
    "tiny_fp32": None,
    "bf16_n1_v131072": dict(n=1, **_BIGV),
    "bf16_n3_v131072": dict(n=3, **_BIGV),
    "bf16_n9_v131072": dict(n=9, **_BIGV),
}


@pytest.fixture(scope="module", params=sorted(CASES))
def tie(request):
    from synth import Workload, get_workload
    kw = CASES[request.param]
    w = get_workload("tiny_fp32") if kw is None else Workload(name="tie_" + request.param,
                                                               tower="tie_" + request.param, **kw)
    case = build_case(w, zero_head=True)
    yield case
    case.dev.close()


def test_zero_head_step0_is_exact(tie):
    w = tie.w
    tok = np.full((w.n, w.B), w.V, dtype=np.int64)
    c = np.zeros((w.n, w.B), bool)
    g = gpu_step(tie, tok, c, GAMMA, want_logits=True)
    log(f"[{w.name}] zero head: conf values {np.unique(g['conf'])}, args {np.unique(g['arg'])}")
    assert (g["z"] == 0).all()
    assert (g["conf"] == np.float32(1.0 / w.V)).all()
    assert (g["arg"] == 0).all()
    expect = np.zeros((w.n, w.B), bool)
    expect[:, 0] = True
    assert np.array_equal(g["U"], expect)
    assert (g["tok"][:, 0] == 0).all() and (g["tok"][:, 1:] == w.V).all()
    # the oracle agrees exactly
    from oracle import oracle_step
    r = oracle_step(tie.orc, tok, c, tie.tau, GAMMA, tie.kv)
    assert (r.conf == 1.0 / w.V).all() and (r.arg == 0).all() and np.array_equal(r.U, expect)


def test_zero_head_mid_block_state(tie):
    """From a state with scattered adopted positions the lowest masked one is adopted."""
    w = tie.w
    rng = np.random.default_rng(3)
    c = rng.random((w.n, w.B)) < 0.4
    c[:, -1] = False   # at least one masked position per sequence
    tok = np.where(c, rng.integers(0, w.V, (w.n, w.B)), w.V)
    g = gpu_step(tie, tok, c, GAMMA)
    first = np.argmax(~c, axis=1)
    expect = np.zeros_like(c)
    expect[np.arange(w.n), first] = True
    assert np.array_equal(g["U"], expect)
    assert (g["conf"][~c] == np.float32(1.0 / w.V)).all() and (g["arg"][~c] == 0).all()
    assert np.array_equal(g["tok"][c], tok[c])   # adopted tokens unchanged


def test_zero_head_block_loop_in_position_order(tie):
    w = tie.w
    torch = tie.torch
    tok = torch.zeros((w.n, w.B), dtype=torch.int32, device="cuda")
    com = torch.zeros((w.n, w.B), dtype=torch.uint8, device="cuda")
    steps = torch.zeros(w.n, dtype=torch.int32, device="cuda")
    cstep = torch.zeros((w.n, w.B), dtype=torch.int8, device="cuda")
    tie.dev.generate_block(tok, com, tie.tau_d, GAMMA, steps=steps, commit_step=cstep)
    tie.dev.sync()
    assert com.cpu().numpy().all()
    assert (tok.cpu().numpy() == 0).all()
    assert (cstep.cpu().numpy() == np.arange(w.B)[None, :]).all()
    assert (steps.cpu().numpy() == w.B).all()
