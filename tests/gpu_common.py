"""Shared pieces of the GPU parity tests: building a case, running steps, comparing.

Parity rules (decisions that rounding can flip are exempt, as listed):
* logits: per row, max_v |z_gpu - z_oracle| / max_v |z_oracle| <= 1e-4 (fp32 towers) or
  2e-2 (bf16 towers), against the plain float64 oracle (the stated bars); and within the
  precision the design carries, 1e-5 (fp32) or 1e-4 (bf16 towers, whose activations enter
  the bf16 matrix cores as a high part plus a remainder: ~2^-17 relative each), so that
  losing the remainder (~5e-3) fails;
* confidences: per masked row, |conf_gpu - conf_oracle| <= conf_oracle * (exp(2 tau delta)
  - 1) + 4e-6 conf_oracle + 1e-7, where delta bounds the row's absolute logit error (the
  measured one where logits are captured, else the design bar times max |z_oracle|):
  the largest scaled logit and the log-sum-exp each move by at most tau * delta, so
  log conf moves by at most 2 tau delta; the last terms cover the fp32 exp and sums;
* token ids and commit masks, each step from the oracle's state, are bit-exact except at
  positions whose oracle confidence is within 1e-3 of gamma or whose oracle top-2 gap
  (p1 - p2) is below 1e-3; a fallback choice is also exempt when the oracle's two most
  confident masked positions differ by less than 1e-3.
"""
from __future__ import annotations

import dataclasses
import os
import sys
from typing import List, Optional

import numpy as np

EXEMPT = 1e-3
LOGIT_BAR = {"f32": 1e-4, "bf16": 2e-2}          # stated bars
LOGIT_DESIGN_BAR = {"f32": 1e-5, "bf16": 1e-4}   # the precision the kernels carry


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@dataclasses.dataclass
class Case:
    w: object
    orc: object
    plens: np.ndarray
    tau: np.ndarray
    kv: object
    dev: object          # Denoiser
    tau_d: object
    torch: object
    keep: object = None


def build_case(w, plens=None, mode=None, device="cuda", zero_head: bool = False) -> Case:
    """The tower of workload w on the device and in the oracle; zero_head replaces the LM
    head by zeros on both sides (every logit exactly 0: the tie cases)."""
    import torch

    from block_diffusion_lm_step_amd import Denoiser
    from synth import draw_inv_temp, draw_prefix_lengths, draw_tower
    from synth.device import prefix_to_device, tower_config, tower_to_device
    from tests.helpers import kv_provider, oracle_weights
    from oracle import OracleTower

    log(f"[case] building {w.name}: n={w.n} B={w.B} d={w.d} L={w.L} V={w.V} dtype={w.dtype} moe={w.moe}")
    tw = draw_tower(w)
    if zero_head:
        tw.lm_head[...] = 0   # +0.0 in float32 and in bf16 bits
    mi = None
    if w.moe:
        from synth import draw_moe
        mi = draw_moe(w)
    plens = draw_prefix_lengths(w) if plens is None else np.asarray(plens, dtype=np.int64)
    tau = draw_inv_temp(w)
    # The GPU carries activations at fp32 precision (no bf16 rounding of activations), so
    # the reference is the plain float64 oracle for every workload.
    mode = mode or "plain"
    orc = OracleTower(oracle_weights(tw, mi), H=w.H, Hkv=w.Hkv, hd=w.hd, eps=w.rms_eps, mode=mode)
    kv = kv_provider(w, plens)
    dW = tower_to_device(tw, device)
    offsets, ks, vs = prefix_to_device(w, plens, device)
    dev = Denoiser(tower_config(w, max_batch=w.n, max_prefix_tokens=max(1, offsets[-1])), dW)
    if mi is not None:
        from synth.device import moe_config, moe_to_device
        dM = moe_to_device(mi, device)
        dev.set_moe(moe_config(w), dM)
        del dM
    dev.set_prefix(offsets, ks, vs)
    del dW
    torch.cuda.synchronize()
    tau_d = torch.from_numpy(tau).to(device)
    return Case(w, orc, plens, tau, kv, dev, tau_d, torch, keep=(ks, vs))


def gpu_step(case: Case, tok: np.ndarray, committed: np.ndarray, gamma: float, want_logits=False):
    """One td_denoise_step from state (tok, committed); returns host arrays."""
    torch = case.torch
    w = case.w
    t_tok = torch.from_numpy(tok.astype(np.int32)).cuda()
    t_c = torch.from_numpy(committed.astype(np.uint8)).cuda()
    newly = torch.zeros_like(t_c)
    conf = torch.full(tok.shape, float("nan"), dtype=torch.float32, device="cuda")
    arg = torch.full(tok.shape, -1, dtype=torch.int32, device="cuda")
    logits = torch.full(tok.shape + (w.V,), float("nan"), dtype=torch.float32, device="cuda") if want_logits else None
    case.dev.denoise_step(t_tok, t_c, case.tau_d, gamma, newly=newly, conf=conf, argmax=arg, logits=logits)
    case.dev.sync()
    out = dict(tok=t_tok.cpu().numpy(), committed=t_c.cpu().numpy().astype(bool), U=newly.cpu().numpy().astype(bool),
               conf=conf.cpu().numpy(), arg=arg.cpu().numpy())
    if want_logits:
        out["z"] = logits.cpu().numpy()
    return out


def logits_rel_err(z_gpu: np.ndarray, z_orc: np.ndarray) -> np.ndarray:
    """Per-row max |dz| / max |z_oracle| over the vocabulary (rows = masked positions)."""
    return np.abs(z_gpu.astype(np.float64) - z_orc).max(axis=-1) / np.abs(z_orc).max(axis=-1)


def decision_mismatches(g: dict, r, committed_in: np.ndarray, gamma: float, rule: int = 0,
                        min_adopt: int = 1) -> List[str]:
    """Non-exempt differences between the GPU step `g` and the oracle StepResult `r`.

    Exempt: predictions whose top-2 probability gap is under EXEMPT; adoptions within
    EXEMPT of gamma; the forced choice (most confident, or the min_adopt-th most
    confident) when the candidates on both sides of it are within EXEMPT.  The
    left-to-right rule involves no floating-point decision and must match exactly."""
    bad = []
    masked = ~committed_in.astype(bool)
    S, B = masked.shape
    for s in range(S):
        conf_o = r.conf[s]
        gap_o = r.gap[s]
        mc = np.where(masked[s], conf_o, -np.inf)
        top = np.sort(mc)[::-1]
        topm = np.sort(conf_o[masked[s]])[::-1]
        fallback_possible = not (mc >= gamma + EXEMPT).any()
        k = min_adopt
        k_tie = (len(topm) > k and topm[k - 1] - topm[k] < EXEMPT and topm[k] < gamma + EXEMPT)
        for p in range(B):
            if not masked[s, p]:
                continue
            near_gamma = abs(conf_o[p] - gamma) < EXEMPT
            if g["arg"][s, p] != r.arg[s, p] and not (gap_o[p] < EXEMPT or near_gamma):
                bad.append(f"seq {s} pos {p}: arg gpu {g['arg'][s, p]} oracle {r.arg[s, p]} "
                           f"(conf {conf_o[p]:.6f}, gap {gap_o[p]:.2e})")
            if g["U"][s, p] != r.U[s, p]:
                if rule == 1:
                    bad.append(f"seq {s} pos {p}: left-to-right commit gpu {g['U'][s, p]} oracle {r.U[s, p]}")
                    continue
                fb_tie = k == 1 and fallback_possible and conf_o[p] >= top[0] - EXEMPT and (
                    top[0] - top[1] < EXEMPT if B > 1 else False)
                rank_tie = k > 1 and k_tie and topm[k] - EXEMPT <= conf_o[p] <= topm[k - 1] + EXEMPT
                if not (near_gamma or fb_tie or rank_tie):
                    bad.append(f"seq {s} pos {p}: commit gpu {g['U'][s, p]} oracle {r.U[s, p]} "
                               f"(conf {conf_o[p]:.6f}, gamma {gamma}, min_adopt {k}, top {topm[:k + 1]})")
    return bad


def conf_abs_err(g: dict, r, committed_in: np.ndarray) -> float:
    masked = ~committed_in.astype(bool)
    if not masked.any():
        return 0.0
    return float(np.abs(g["conf"][masked].astype(np.float64) - r.conf[masked]).max())


def check_logits(err: np.ndarray, dtype: str, what: str = "") -> None:
    """Per-row relative logit errors against the stated bar and the design bar."""
    assert err.max() <= LOGIT_BAR[dtype], f"{what} logits rel err {err.max():.3e} > {LOGIT_BAR[dtype]}"
    assert err.max() <= LOGIT_DESIGN_BAR[dtype], \
        f"{what} logits rel err {err.max():.3e} > design bar {LOGIT_DESIGN_BAR[dtype]}"


def conf_violations(g: dict, r, committed_in: np.ndarray, tau: np.ndarray, dtype: str,
                    z_gpu: Optional[np.ndarray] = None, z_orc: Optional[np.ndarray] = None) -> List[str]:
    """Masked rows whose GPU confidence is outside the bound derived from the logit error.

    delta per row: the measured max |z_gpu - z_oracle| when both logit arrays ([S][B][V])
    are given, else LOGIT_DESIGN_BAR * max |z_oracle| (r.zmax)."""
    masked = ~committed_in.astype(bool)
    if z_gpu is not None and z_orc is not None:
        delta = np.where(masked, np.abs(np.nan_to_num(z_gpu.astype(np.float64) - z_orc)).max(axis=-1), np.nan)
    else:
        delta = LOGIT_DESIGN_BAR[dtype] * r.zmax
    out = []
    for s, p in zip(*np.nonzero(masked)):
        co, cg = float(r.conf[s, p]), float(g["conf"][s, p])
        bound = co * (np.expm1(2.0 * float(tau[s, p]) * float(delta[s, p])) + 4e-6) + 1e-7
        if not abs(cg - co) <= bound:
            out.append(f"seq {s} pos {p}: conf gpu {cg:.8f} oracle {co:.8f} (|d| {abs(cg - co):.2e} > {bound:.2e}, "
                       f"tau {float(tau[s, p]):.2f}, delta {float(delta[s, p]):.2e})")
    return out
