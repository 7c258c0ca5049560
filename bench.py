#!/usr/bin/env python3
"""Benchmark of the block-diffusion denoising loop on one MI355X.

A bench "step" is one pass of the whole hot path over one batch: td_generate_block, the
device-driven loop of denoising steps (embedding, L layers of fused QKV / split-K
attention / output / MLP projections, LM head with the fused vocabulary reduction,
on-device commit) from an all-[MASK] block until every position of every sequence is
adopted.  The loop is enqueued whole (no issue window): no host round trip inside it.

Default workload: the largest single-GPU configuration, the throughput sweep at block 32
(batch 64, prefixes uniform in [1024, 4096], the d 2048 bf16 tower, vocabulary 131072,
gamma 0.8).  Inputs are synthetic and resident in HBM before the timed region.  Prints
one JSON line; with --workloads a,b,... one line per workload.

Measurement:
* value: committed tokens/s = timed blocks x n x B / wall time of the timed region;
* a profiling pass (HIP events around every launch of every kernel class, on the ctx's
  stream) gives each class's time, and the algorithmic work of each launch follows from
  the step it belongs to: the sequences still active at that step (their prefix K/V, their
  rows in the layer GEMMs) and the rows still masked (the LM head), read off the block's
  own step counts and adoption steps;
* roofline: the kernel class with the most time, re-measured with events inside the timed
  region, against its own bound (bytes against HBM, or FLOPs against the bf16 matrix
  cores, whichever takes longer at peak);
* peaks: the published ones and the chip's own (td_measure_peaks).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores, published
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 (matrix and vector), published
METRIC = "committed tokens/s + denoise steps/s, 1 GPU; % of HBM / MFMA roofline"
DEFAULT_WORKLOAD = "sweep64_b32"

# Kernel classes of the profiling tags (td.h td_prof_kind) and the projections of TD_PROF_GEMM.
K_LMHEAD, K_GEMM, K_ATTN, K_STEP, K_MOE, K_MERGE, K_COMMIT, K_EMBED = 1, 2, 3, 4, 5, 6, 7, 8
PROJ = ("qkv", "out", "mlp_up", "mlp_down", "router")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20, help="timed blocks")
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--workloads", default=None,
                   help="comma-separated workloads, one JSON line each (overrides --workload)")
    p.add_argument("--gamma", type=float, default=None)
    p.add_argument("--profile-blocks", type=int, default=2, help="blocks of the per-class profiling pass")
    p.add_argument("--window-compare", type=int, default=2,
                   help="also time the blocks with td_set_issue_window(W) (the host stops enqueuing steps once "
                        "the device reports the batch adopted; it polls a host word); 0: skip")
    p.add_argument("--cpu-seconds", type=float, default=30.0,
                   help="budget of the CPU oracle sample (whole-batch step 0, then whole block loops)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-peaks", action="store_true")
    p.add_argument("--step0", type=int, default=0,
                   help="profiling mode: K denoising steps from the all-[MASK] state (every sequence active, every "
                        "row masked) instead of block loops; prints the per-class record of those steps")
    p.add_argument("--ar", type=int, default=0,
                   help="also time K steps of AR decoding (td_ar_step on a block-size-1 ctx), reported under 'ar'")
    p.add_argument("--blocks", type=int, default=0,
                   help="also time K consecutive blocks of multi-block generation, reported under 'multiblock'")
    p.add_argument("--calibrate-copy-mb", type=int, default=0,
                   help="before the timed region, one elementwise copy of this many MiB (the scale of the HBM "
                        "byte counters)")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="no benchmark: turn the counter CSVs of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; "
                        "both of --step0 runs with --calibrate-copy-mb) into the HBM traffic record of "
                        "--traffic-kernel under profiles/")
    p.add_argument("--traffic-kernel", default="attention",
                   help="class of the traffic record: attention, lm_head or gemm_<qkv|out|mlp_up|mlp_down>")
    return p.parse_args(argv)


# ----------------------------------------------------------------------------- kernel classes

def class_name(kind: int, sub: int) -> str:
    if kind == K_GEMM:
        return "gemm_" + PROJ[sub]
    if kind == K_MOE:
        return ("moe_up", "moe_down")[sub]
    return {K_LMHEAD: "lm_head", K_ATTN: "attention", K_MERGE: "attn_merge", K_COMMIT: "commit",
            K_EMBED: "embed"}[kind]


def class_kind(name: str):
    if name.startswith("gemm_"):
        return K_GEMM, PROJ.index(name[5:])
    if name.startswith("moe_"):
        return K_MOE, ("moe_up", "moe_down").index(name)
    return {"lm_head": K_LMHEAD, "attention": K_ATTN, "attn_merge": K_MERGE, "commit": K_COMMIT,
            "embed": K_EMBED}[name], 0


def kernel_label(w, cls: str) -> str:
    """The kernel the library plans for class cls on workload w at its first step."""
    M = w.n * w.B
    tiled = w.dtype == "bf16" and M >= 128
    if cls == "attention":
        R = w.G * w.B
        if R <= 16:
            return "attn_direct_kernel (one 16-row tile, pages straight to registers)"
        if R <= 32:
            return "attn_direct_kernel (two 16-row tiles, pages straight to registers)"
        return "attn_group_kernel (grouped-query rows, pages staged in LDS)"
    if cls == "lm_head":
        if tiled:
            return "gemm_tile_kernel<VSTAT> (LM head in MFMA tiles + fused tau-scaled vocab max/sumexp/argmax)"
        if w.dtype == "bf16" and M <= 16 and w.d <= 2048:
            return "lmhead_lds_kernel (LM head, activations staged in LDS, fused vocab max/sumexp/argmax)"
        return "lmhead_kernel (LM head over the row list, fused vocab max/sumexp/argmax)"
    if cls.startswith("gemm_"):
        return ("gemm_tile_kernel (MFMA tiles through LDS)" if tiled else "gemm_wk_kernel (weight streaming)") + \
            f": {cls[5:]} projection"
    return cls


def class_work(w, plens, cls: str, act: np.ndarray, masked_rows: int, moe_active: float = 0.0):
    """(bytes, flops) of one launch of class cls at a step whose active sequences are act
    (bool [n]) with masked_rows rows still masked.  Algorithmic: every weight or cache byte
    once, the rows that need computing (active sequences; masked rows for the LM head)."""
    elt = 2 if w.dtype == "bf16" else 4
    nact = int(act.sum())
    if cls.startswith("gemm_"):
        N, K = {"qkv": (w.qkv_dim, w.d), "out": (w.d, w.H * w.hd), "mlp_up": (w.F, w.d),
                "mlp_down": (w.d, w.F), "router": ((w.moe[0] + 31) // 32 * 32 if w.moe else 0, w.d)}[cls[5:]]
        return N * K * elt, 2 * w.B * nact * N * K
    if cls == "attention":
        P = plens[act].astype(np.float64)
        return float(P.sum()) * 2 * w.Hkv * w.hd * elt, float((4.0 * w.B * (P + w.B) * w.hd * w.H).sum())
    if cls == "lm_head":
        return w.V * w.d * elt, 2.0 * masked_rows * w.V * w.d
    if cls in ("moe_up", "moe_down"):
        return moe_active * w.moe[3] * w.d * elt, 2.0 * w.B * nact * w.moe[1] * w.moe[3] * w.d
    return 0.0, 0.0


def mfma_peak(w) -> float:
    return BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS


def floor_ms(w, nbytes: float, flops: float) -> float:
    return max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (mfma_peak(w) * 1e12)) * 1e3


def step_activity(steps: np.ndarray, cstep: np.ndarray):
    """Per step t of the block loop: active sequences (steps[s] > t) and rows still masked
    on entry (adopted at step t or later)."""
    S = int(steps.max())
    return [(steps > t, int((cstep >= t).sum())) for t in range(S)]


def summarize(w, plens, records, activity, B: int, moe_active: float = 0.0):
    """Per-class totals over the working launches of a tagged profile of whole blocks
    issued B steps each (records: [(ms, (kind, sub, layer))] in launch order; a step starts
    at its embedding launch)."""
    S = len(activity)
    out, empty_ms, t_glob = {}, 0.0, -1
    for ms, (kind, sub, layer) in records:
        if kind == K_EMBED:
            t_glob += 1
        t = t_glob % B
        if t >= S:            # a step after the batch is adopted: every launch exits at once
            empty_ms += ms
            continue
        cls = class_name(kind, sub)
        nb, fl = class_work(w, plens, cls, *activity[t], moe_active=moe_active)
        r = out.setdefault(cls, dict(ms=0.0, launches=0, bytes=0.0, flops=0.0, floor_ms=0.0))
        r["ms"] += ms
        r["launches"] += 1
        r["bytes"] += nb
        r["flops"] += fl
        r["floor_ms"] += floor_ms(w, nb, fl)
    nblocks = (t_glob + 1) // B
    return out, empty_ms, max(1, nblocks)


def roofline_of(w, cls: str, r: dict, peaks: dict) -> dict:
    """Bound, achieved rate and fraction of one class from its totals r."""
    hbm_ms = r["bytes"] / (HBM_PEAK_GBS * 1e9) * 1e3
    mfma_ms = r["flops"] / (mfma_peak(w) * 1e12) * 1e3
    sec = r["ms"] * 1e-3
    if r["bytes"] == 0 and r["flops"] == 0:
        out = dict(bound="latency", achieved=None, peak=None, unit=None, frac=None)
    elif mfma_ms > hbm_ms:
        ach = r["flops"] / sec / 1e12
        out = dict(bound="mfma", achieved=round(ach, 1), peak=mfma_peak(w), unit="TFLOP/s",
                   frac=round(ach / mfma_peak(w), 4))
        meas = peaks.get("mfma_bf16_tflops") if w.dtype == "bf16" else None
        if meas:
            out["frac_of_measured_peak"] = round(ach / meas, 4)
        if w.dtype == "bf16" and cls != "attention":
            # the activations enter the bf16 matrix cores as a high part plus a remainder
            out["issued_frac"] = round(2 * ach / mfma_peak(w), 4)
    else:
        ach = r["bytes"] / sec / 1e9
        out = dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(ach / HBM_PEAK_GBS, 4))
        if peaks.get("hbm_read_gbs"):
            out["frac_of_measured_peak"] = round(ach / peaks["hbm_read_gbs"], 4)
    n = max(1, r["launches"])
    out.update(kernel=kernel_label(w, cls), cls=cls, floor_frac=round(r["floor_ms"] / r["ms"], 4) if r["ms"] else None,
               alg_bytes_per_launch=round(r["bytes"] / n), alg_flops_per_launch=round(r["flops"] / n),
               avg_launch_ms=round(r["ms"] / n, 5), launches_averaged=r["launches"])
    return out


# ----------------------------------------------------------------------------- HBM traffic records

TRAFFIC_SOURCES = {
    "attention": ("k_attn.hip", "td_device.h", "td_kernels.h", "td_api.cpp"),   # td_api: the work items
    "lm_head": ("k_gemm.hip", "k_gemm_tile.hip", "td_device.h", "td_kernels.h"),
    "gemm": ("k_gemm_tile.hip", "k_gemm_wk.hip", "td_device.h", "td_kernels.h"),
}
# Kernel-name substrings of each class in a rocprofv3 counter CSV.
TRAFFIC_NAMES = {"attention": ("attn_direct_kernel", "attn_group_kernel"),
                 "lm_head": ("lmhead_lds_kernel", "lmhead_kernel", "gemm_tile_kernel<3,"),
                 "gemm": ("gemm_tile_kernel", "gemm_wk_kernel")}


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "block_diffusion_lm_step_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_family(cls: str) -> str:
    return "gemm" if cls.startswith("gemm_") else cls


def traffic_path(workload: str, cls: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{traffic_family(cls)}_{workload}.json")


def traffic_record(workload: str, cls: str):
    """HBM bytes over algorithmic bytes of class cls's full-batch launches, from the
    rocprofv3 counters, if they were taken on the current sources of that class."""
    fam = traffic_family(cls)
    if fam not in TRAFFIC_SOURCES:
        return None
    try:
        with open(traffic_path(workload, cls)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != source_hash(*TRAFFIC_SOURCES[fam]):
        return None
    return rec


def write_traffic(workload: str, cls: str, fetch_csv: str, write_csv: str, calib_mb: int, alg_bytes: float) -> dict:
    """Counter values per dispatch (KiB) -> bytes, scaled by the calibration copy.

    The elementwise copy of calib_mb MiB reads and writes exactly that many bytes; the ratio
    of that size to what FETCH_SIZE / WRITE_SIZE report for it scales the class's readings.
    Dispatches that exited early (nothing to do) read ~nothing and are left out."""
    import csv

    fam = traffic_family(cls)
    names = TRAFFIC_NAMES[fam]

    def per_dispatch(path, counter):
        ks, blit, elem = [], [], []
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                v = float(row["Counter_Value"]) * 1024.0
                k = row["Kernel_Name"]
                if any(n in k for n in names):
                    ks.append(v)
                elif "copyBuffer" in k:
                    blit.append(v)
                elif "MulFunctor" in k:
                    elem.append(v)
        return ks, blit, elem

    calib = calib_mb * 1024 * 1024
    out = {}
    for name, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        ks, blit, elem = per_dispatch(path, counter)
        if not ks or not elem:
            raise SystemExit(f"{path}: no {fam} or calibration dispatches with {counter}")
        factor = calib / max(elem)
        work = sorted(v for v in ks if v > 0.5 * max(ks)) if name == "fetch" else sorted(ks)
        raw = float(np.median(work))
        out[name] = dict(counter=counter, raw_bytes_per_launch=raw, calibration_kernel="elementwise (16 B per lane)",
                         calibration_raw_bytes=max(elem), factor=factor, bytes_per_launch=raw * factor,
                         dispatches=len(work), blit_copy_raw_bytes=max(blit) if blit else None)
    hbm = out["fetch"]["bytes_per_launch"] + out["write"]["bytes_per_launch"]
    rec = dict(cls=cls, kernel_names=list(names), workload=workload,
               source_sha256_16=source_hash(*TRAFFIC_SOURCES[fam]), calibration_copy_bytes=calib,
               fetch=out["fetch"], write=out["write"], hbm_bytes_per_launch=hbm, alg_bytes_per_launch=alg_bytes,
               ratio=hbm / alg_bytes if alg_bytes else None)
    os.makedirs(os.path.dirname(traffic_path(workload, cls)), exist_ok=True)
    with open(traffic_path(workload, cls), "w") as f:
        json.dump(rec, f, indent=1)
    return rec


# ----------------------------------------------------------------------------- CPU baseline

def cpu_baseline(w, budget_s: float, batch_step0: bool = True):
    """The oracle as it stands, on this host's cores, on a bounded sample of the workload:
    for a batch of more than four sequences, one step of the whole batch from all-[MASK];
    then whole block loops on the first (at most four) sequences until min(budget, 10 s)."""
    from oracle import OracleTower, oracle_step
    from synth import draw_inv_temp, draw_prefix_lengths, draw_tower, f32_from_bf16_bits
    from synth.gen import draw_prefix_kv

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        threads = os.cpu_count()
    tw = draw_tower(w)
    f = tw.as_f32
    W = dict(tok_emb=f(tw.tok_emb), pos_emb=f(tw.pos_emb), final_norm=f(tw.final_norm), lm_head=f(tw.lm_head),
             wq=[f(a) for a in tw.wq], wk=[f(a) for a in tw.wk], wv=[f(a) for a in tw.wv], wo=[f(a) for a in tw.wo],
             w1=[f(a) for a in tw.w1], w2=[f(a) for a in tw.w2], attn_norm=[f(a) for a in tw.attn_norm],
             mlp_norm=[f(a) for a in tw.mlp_norm])
    del tw
    if w.moe:   # the mixture of experts, widened to float32 (the oracle reads it expert by expert)
        from synth import draw_moe
        mi = draw_moe(w)
        W["moe"] = dict(top_k=w.moe[1], router=[f(a) for a in mi.router], w1=[f(a) for a in mi.w1],
                        w2=[f(a) for a in mi.w2], sw1=[f(a) for a in mi.sw1], sw2=[f(a) for a in mi.sw2])
        del mi
    orc = OracleTower(W, H=w.H, Hkv=w.Hkv, hd=w.hd, eps=w.rms_eps, mode="plain")
    plens = draw_prefix_lengths(w)
    tau = draw_inv_temp(w)
    n_s = min(w.n, 4)   # sequences of the block-loop sample (all of a batch-1 workload)
    whole = batch_step0 and w.n > n_s
    cache = {}

    def kv(l, s):
        if (l, s) not in cache:
            k = draw_prefix_kv(w, l, s, int(plens[s]), "k")
            v = draw_prefix_kv(w, l, s, int(plens[s]), "v")
            if w.dtype == "bf16":
                k, v = f32_from_bf16_bits(k), f32_from_bf16_bits(v)
            cache[(l, s)] = (k, v)
        return cache[(l, s)]

    for l in range(w.L):   # inputs staged and weights widened before timing, as td_create is untimed
        for s in range(w.n if whole else n_s):
            kv(l, s)
        for name in ("wq", "wk", "wv", "wo", "attn_norm", "mlp_norm") + (() if w.moe else ("w1", "w2")):
            orc._w(name, l)
    for name in ("lm_head", "pos_emb", "final_norm"):
        orc._w(name)
    out = {}
    if whole:
        tok = np.full((w.n, w.B), w.V, dtype=np.int64)
        t0 = time.perf_counter()
        r = oracle_step(orc, tok, np.zeros((w.n, w.B), bool), tau, w.gamma, kv)
        dt0 = time.perf_counter() - t0
        out["batch_step0"] = dict(seconds=round(dt0, 3), sequences=w.n, positions_adopted=int(r.U.sum()),
                                  denoise_steps_per_s=round(1.0 / dt0, 5))
        for key in [k for k in cache if k[1] >= n_s]:
            del cache[key]
    # Whole block loops from all-[MASK], repeated until at least min(budget, 10 s) of work;
    # a loop still running at the budget is cut there (its adopted positions count).
    min_s = min(budget_s, 10.0)
    t0 = time.perf_counter()
    steps = committed = blocks = 0
    while True:
        tok = np.full((n_s, w.B), w.V, dtype=np.int64)
        c = np.zeros((n_s, w.B), bool)
        while not c.all() and time.perf_counter() - t0 < budget_s:
            r = oracle_step(orc, tok, c, tau[:n_s], w.gamma, kv)
            committed += int(r.U.sum())
            steps += 1
            tok, c = r.tok, r.committed
        blocks += int(c.all())
        if not c.all() or time.perf_counter() - t0 >= min_s:
            break
    dt = time.perf_counter() - t0
    sample = (f"{steps} oracle steps: {blocks} whole block loop(s) from all-[MASK]"
              f"{'' if c.all() else ' and one cut at the time budget'} on sequences 0..{n_s - 1} of {w.name} "
              f"(float64 numpy, BLAS on {threads} threads), {committed} positions adopted")
    if whole:
        sample += f"; before them one step of the whole batch of {w.n} sequences (batch_step0)"
    out.update(value=committed / dt, unit="committed tokens/s", cores=int(threads), nproc=os.cpu_count(),
               kind="oracle", sample=sample, denoise_steps_per_s=steps / dt, seconds=dt)
    return out


# ----------------------------------------------------------------------------- the GPU runs

class Inputs:
    """Device tensors of one workload (towers and prefixes shared between workloads that
    share their streams)."""
    towers: dict = {}
    prefixes: dict = {}


def setup(w, room: int = 0):
    import torch

    from block_diffusion_lm_step_amd import Denoiser
    from synth import draw_inv_temp, draw_prefix_lengths, draw_tower
    from synth.device import prefix_to_device, tower_config, tower_to_device

    key = (w.tower, w.B, bool(w.moe))
    if key not in Inputs.towers:
        Inputs.towers.clear()
        torch.cuda.empty_cache()
        Inputs.towers[key] = tower_to_device(draw_tower(w))
    plens = draw_prefix_lengths(w)
    pkey = (w.batch, w.L, room)
    if pkey not in Inputs.prefixes:
        Inputs.prefixes.clear()
        torch.cuda.empty_cache()
        Inputs.prefixes[pkey] = prefix_to_device(w, plens, room=room)
    offsets, ks, vs = Inputs.prefixes[pkey]
    tau = torch.from_numpy(draw_inv_temp(w)).cuda()
    dev = Denoiser(tower_config(w, max_batch=w.n, max_prefix_tokens=max(1, offsets[-1] + room * w.n)),
                   Inputs.towers[key])
    if w.moe:   # every layer's MLP a mixture of experts
        from synth import draw_moe
        from synth.device import moe_config, moe_to_device
        dM = moe_to_device(draw_moe(w))
        dev.set_moe(moe_config(w), dM)
        del dM
    dev.set_prefix(offsets, ks, vs)
    torch.cuda.synchronize()
    return dev, plens, tau


def time_ar(args, w, plens) -> dict:
    """K greedy AR decoding steps of the context tower (with its own final norm and LM
    head) on a ctx of block size 1 over the same prefix: one token per sequence per step,
    each step appending the token's K/V.  The binding is reset before each repetition."""
    import torch

    from block_diffusion_lm_step_amd import Denoiser
    from synth import draw_tower
    from synth.device import cache_pages, prefix_to_device, tower_config, tower_to_device

    K = args.ar
    w1 = w.with_(B=1)
    _, ks, vs = prefix_to_device(w1, plens, room=K)
    caps = cache_pages(plens, K)
    dev = Denoiser(tower_config(w1, max_batch=w.n, max_prefix_tokens=int(plens.sum()) + K * w.n),
                   tower_to_device(draw_tower(w1)))
    dev.set_context_tower(tower_to_device(draw_tower(w1, context=True, ar_head=True)))
    lengths = [int(p) for p in plens]
    tok = torch.zeros(w.n, dtype=torch.int32, device="cuda")

    def run():
        dev.bind_cache(lengths, caps, ks, vs)
        tok.fill_(1)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(K):
            dev.ar_step(tok)
        dev.sync()
        return time.perf_counter() - t

    run()
    reps = 3
    el = sum(run() for _ in range(reps)) / reps
    dev.close()
    log(f"[bench] AR: {K} steps in {el * 1e3:.2f} ms")
    return dict(steps=K, value=round(K * w.n / el, 3), unit="tokens/s", ms_per_token_step=round(el * 1e3 / K, 4),
                timing="host clock around K td_ar_step calls and one sync")


def time_multiblock(args, w, plens, tau, dev, tok, com, steps) -> dict:
    """K consecutive blocks of multi-block generation on caches bound with room for them:
    each block is generated, then the context tower appends its K/V to the prefix.  The
    binding is reset to the original prefix before each timed repetition."""
    import torch

    from synth import draw_tower
    from synth.device import cache_pages, prefix_to_device, tower_to_device

    K = args.blocks
    room = K * w.B
    _, ks, vs = prefix_to_device(w, plens, room=room)
    caps = cache_pages(plens, room)
    dev.set_context_tower(tower_to_device(draw_tower(w, context=True)))
    lengths = [int(p) for p in plens]

    def run():
        dev.bind_cache(lengths, caps, ks, vs)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(K):
            dev.generate_block(tok, com, tau, w.gamma, steps=steps)
            dev.append_block(tok)
        dev.sync()
        return time.perf_counter() - t

    run()
    reps = 3
    el = sum(run() for _ in range(reps)) / reps
    log(f"[bench] multi-block: {K} blocks in {el * 1e3:.2f} ms")
    return dict(blocks=K, value=round(K * w.n * w.B / el, 3), unit="committed tokens/s",
                ms_per_block=round(el * 1e3 / K, 4),
                timing="host clock around K (td_generate_block, td_append_block) pairs and one sync")


def measure_peaks() -> dict:
    import torch

    from block_diffusion_lm_step_amd import measure_peaks as mp
    buf = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")   # 2 GiB: far beyond the 256 MB last-level cache
    p = mp(buf)
    del buf
    torch.cuda.empty_cache()
    return {k: round(v, 1) for k, v in p.items()}


def bench_workload(args, w, peaks: dict, want_cpu: bool) -> dict:
    import torch

    from block_diffusion_lm_step_amd import TD_PROF_ATTENTION, TD_PROF_ATTN_MERGE, TD_PROF_COMMIT, TD_PROF_EMBED, \
        TD_PROF_GEMM, TD_PROF_LMHEAD, TD_PROF_MOE

    log(f"[bench] workload {w.name}: n={w.n} B={w.B} d={w.d} H={w.H}/{w.Hkv}x{w.hd} L={w.L} F={w.F} V={w.V} "
        f"gamma={w.gamma}")
    t = time.time()
    dev, plens, tau = setup(w)
    log(f"[bench] inputs resident in HBM ({time.time() - t:.1f} s)")
    tok = torch.zeros((w.n, w.B), dtype=torch.int32, device="cuda")
    com = torch.zeros((w.n, w.B), dtype=torch.uint8, device="cuda")
    steps = torch.zeros(w.n, dtype=torch.int32, device="cuda")
    cstep = torch.zeros((w.n, w.B), dtype=torch.int8, device="cuda")
    all_kinds = (TD_PROF_LMHEAD, TD_PROF_GEMM, TD_PROF_ATTENTION, TD_PROF_ATTN_MERGE, TD_PROF_COMMIT, TD_PROF_EMBED) + \
        ((TD_PROF_MOE,) if w.moe else ())

    def block():
        dev.generate_block(tok, com, tau, w.gamma, steps=steps, commit_step=cstep)

    if args.step0:
        return step0_record(args, w, dev, plens, tau, tok, com, all_kinds, peaks)

    dev.set_issue_window(0)
    for _ in range(args.warmup):
        block()
    dev.sync()
    st0, cs0 = steps.cpu().numpy().copy(), cstep.cpu().numpy().copy()
    activity = step_activity(st0, cs0)
    S = len(activity)
    if args.calibrate_copy_mb > 0:
        nb = args.calibrate_copy_mb * 1024 * 1024
        src = torch.ones(nb // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    log("[bench] warmup done")

    # Profiling pass: every class bracketed, whole blocks of B issued steps.
    moe_active = 0.0
    if w.moe:
        dev.moe_stats()
    dev.profile_begin(*all_kinds)
    for _ in range(args.profile_blocks):
        block()
    ms, tags = dev.profile_end(tags=True)
    if w.moe:
        launches, act = dev.moe_stats()
        moe_active = act / max(1, launches)
    classes, empty_ms, nblk = summarize(w, plens, list(zip(ms, tags)), activity, w.B, moe_active)
    dominant = max((c for c in classes if classes[c]["bytes"] or classes[c]["flops"]), key=lambda c: classes[c]["ms"])
    dkind, dsub = class_kind(dominant)

    # Timed region: blocks enqueued whole; events on the dominant class only, and for a
    # per-layer class on its middle layer only (one pair of events per step, as for the
    # LM head: more events between short launches would slow the loop they time).
    per_step_launches = 1
    if dkind != K_LMHEAD:
        dev.profile_layer(w.L // 2)
    dev.profile_begin(dkind)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        block()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dms, dtags = dev.profile_end(tags=True)
    dev.profile_layer(-1)
    dev.sync()
    elapsed = t1 - t0
    st, cs = steps.cpu().numpy(), cstep.cpu().numpy()
    assert com.cpu().numpy().all(), "block not fully committed"
    assert np.array_equal(st, st0) and np.array_equal(cs, cs0), "blocks differ between runs"
    log(f"[bench] {args.steps} blocks in {elapsed * 1e3:.2f} ms; {S} steps per block; dominant class {dominant}")
    dom = dict(ms=0.0, launches=0, bytes=0.0, flops=0.0, floor_ms=0.0)
    i = 0
    for d_ms, (kind, sub, layer) in zip(dms, dtags):
        if kind != dkind:
            continue
        if kind in (K_GEMM, K_MOE) and sub != dsub:
            continue
        t_step = (i // per_step_launches) % w.B
        i += 1
        if t_step >= S:
            continue
        nb, fl = class_work(w, plens, dominant, *activity[t_step], moe_active=moe_active)
        dom["ms"] += d_ms
        dom["launches"] += 1
        dom["bytes"] += nb
        dom["flops"] += fl
        dom["floor_ms"] += floor_ms(w, nb, fl)
    roof = roofline_of(w, dominant, dom, peaks)
    rec = traffic_record(w.name, dominant)
    roof["traffic"] = round(rec["ratio"] * roof["alg_bytes_per_launch"]) if rec and rec.get("ratio") else None
    if rec:
        roof["traffic_ratio_full_batch"] = round(rec["ratio"], 4)

    block_ms = elapsed / args.steps * 1e3
    kernels = []
    for c, r in sorted(classes.items(), key=lambda kv: -kv[1]["ms"]):
        k = roofline_of(w, c, r, peaks)
        k["ms_per_block"] = round(r["ms"] / nblk, 4)
        k["share_of_block"] = round(r["ms"] / nblk / block_ms, 4)
        kernels.append(k)
    block_floor = sum(r["floor_ms"] for r in classes.values()) / nblk

    out = {
        "metric": METRIC,
        "value": round(args.steps * w.n * w.B / elapsed, 3),
        "unit": "committed tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(block_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; random-init tower weights N(0,0.02), prefix K/V N(0,1))",
        "config": {"workload": w.name, "batch": w.n, "prefix_tokens": int(plens.sum()), "block": w.B, "gamma": w.gamma,
                   "issue_window": 0, "d_model": w.d, "heads": w.H, "kv_heads": w.Hkv, "head_dim": w.hd,
                   "layers": w.L, "d_ff": w.F, "vocab": w.V,
                   **({"moe": {"experts": w.moe[0], "top_k": w.moe[1], "shared": w.moe[2],
                               "d_expert": w.moe[3]}} if w.moe else {})},
        "step_is": "one block loop (td_generate_block) over the whole batch; ms_per_step is per block",
        "denoise_steps_per_s": round(args.steps * S / elapsed, 3),
        "denoise_steps_per_block": S,
        "ms_per_denoise_step": round(block_ms / S, 4),
        "sequence_steps_histogram": {int(k): int(v) for k, v in zip(*np.unique(st, return_counts=True))},
        "roofline": roof,
        "roofline_kernels": kernels,
        "block_floor_ms": round(block_floor, 4),
        "block_roofline_frac": round(block_floor / block_ms, 4),
        "empty_steps_ms_per_block": round(empty_ms / nblk, 4),
        "peaks": {"published": {"hbm_gbs": HBM_PEAK_GBS, "bf16_mfma_tflops": BF16_PEAK_TFLOPS},
                  "measured": peaks or None},
    }
    if args.window_compare > 0:
        dev.set_issue_window(args.window_compare)
        block()
        dev.sync()
        torch.cuda.synchronize()
        a = time.perf_counter()
        for _ in range(args.steps):
            block()
        torch.cuda.synchronize()
        el = time.perf_counter() - a
        dev.set_issue_window(0)
        out[f"issue_window_{args.window_compare}"] = dict(
            value=round(args.steps * w.n * w.B / el, 3), ms_per_block=round(el / args.steps * 1e3, 4),
            note="the host enqueues step s once the device reports step s - W finished (it polls a word of pinned "
                 "host memory) and stops once the batch is adopted")
    if args.blocks > 0:
        out["multiblock"] = time_multiblock(args, w, plens, tau, dev, tok, com, steps)
    if args.ar > 0:
        ar = time_ar(args, w, plens)
        ar["diffusion_to_ar"] = round((out["multiblock"]["value"] if "multiblock" in out else out["value"])
                                      / ar["value"], 4)
        out["ar"] = ar
    dev.close()
    if want_cpu:
        log("[bench] timing the CPU oracle sample")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    return out


def step0_record(args, w, dev, plens, tau, tok, com, all_kinds, peaks) -> dict:
    """K steps from the all-[MASK] state (full batch, every row masked): the shape the
    rocprofv3 summaries are taken on.  Per-class averages from the tagged events."""
    import torch

    def step():
        tok.fill_(w.V)
        com.zero_()
        dev.denoise_step(tok, com, tau, w.gamma)

    for _ in range(max(1, args.warmup)):
        step()
    dev.sync()
    if args.calibrate_copy_mb > 0:
        nb = args.calibrate_copy_mb * 1024 * 1024
        src = torch.ones(nb // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    act = [(np.ones(w.n, bool), w.n * w.B)]
    dev.profile_begin(*all_kinds)
    for _ in range(args.step0):
        step()
    ms, tags = dev.profile_end(tags=True)
    torch.cuda.synchronize()
    a = time.perf_counter()
    for _ in range(args.step0):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - a
    classes, _, _ = summarize(w, plens, list(zip(ms, tags)), act, 1)
    kernels = []
    for c, r in sorted(classes.items(), key=lambda kv: -kv[1]["ms"]):
        k = roofline_of(w, c, r, peaks)
        k["ms_per_step"] = round(r["ms"] / args.step0, 4)
        kernels.append(k)
    dev.close()
    return dict(mode="step0", workload=w.name, steps=args.step0, ms_per_step=round(el / args.step0 * 1e3, 4),
                step_floor_ms=round(sum(r["floor_ms"] for r in classes.values()) / args.step0, 4),
                roofline_kernels=kernels, peaks=peaks or None)


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the library has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    from synth import get_workload

    if args.traffic_from:
        if args.calibrate_copy_mb <= 0:
            raise SystemExit("--traffic-from needs the --calibrate-copy-mb the counter runs used")
        w = get_workload(args.workload)
        plens = __import__("synth").draw_prefix_lengths(w)
        nb, _ = class_work(w, plens, args.traffic_kernel, np.ones(w.n, bool), w.n * w.B)
        print(json.dumps(write_traffic(w.name, args.traffic_kernel, *args.traffic_from, args.calibrate_copy_mb, nb)))
        return
    import torch  # noqa: F401

    peaks = {} if args.no_peaks else measure_peaks()
    if peaks:
        log(f"[bench] measured peaks: {peaks}")
    names = args.workloads.split(",") if args.workloads else [args.workload]
    for name in names:
        w = get_workload(name)
        if args.gamma is not None:
            w = w.with_(gamma=args.gamma)
        out = bench_workload(args, w, peaks, want_cpu=not args.no_cpu_baseline and not args.step0)
        print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
