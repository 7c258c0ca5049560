#!/usr/bin/env python3
"""Benchmark of the block-diffusion denoising loop on one MI355X.

A bench "step" is one pass of the whole hot path over one batch: td_generate_block, i.e.
the device-driven loop of denoising steps (embedding, L layers of fused QKV / split-K
attention / output / MLP projections, LM head with fused vocab reduction, on-device
commit) that starts from an all-[MASK] block and ends when every position is adopted.

Default workload: bf16 tower at batch 1 (prefix 4096, d 2048, 16 x 128 heads, 8 layers,
MLP 8192, vocab 131072, block 16, gamma 0.8), inputs synthetic and resident in HBM
before the timed region.  The loop is issued with a window of 2 steps
(td_set_issue_window): steps after the device reports the block adopted are not
enqueued; --issue-window 0 enqueues all B at once.  Prints one JSON line.
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
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
METRIC = "committed tokens/s + denoise steps/s, 1 GPU; % of HBM / MFMA roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50, help="timed blocks")
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="b1_p4096")
    p.add_argument("--gamma", type=float, default=None)
    p.add_argument("--cpu-seconds", type=float, default=20.0,
                   help="budget of the CPU oracle sample: whole block loops until min(budget, 10 s) has passed, "
                        "none running past the budget")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--issue-window", type=int, default=2,
                   help="td_set_issue_window: step s is enqueued once the device has finished step s - W, none "
                        "after it reports the batch adopted (0: the whole block loop at once)")
    p.add_argument("--breakdown", action="store_true", help="also time each kernel class (extra blocks)")
    p.add_argument("--ar", type=int, default=0,
                   help="also time K steps of AR decoding (td_ar_step: the context tower with its own head, one "
                        "token per sequence per step) on a block-size-1 ctx: reported under 'ar', with the ratio "
                        "of the block rate to it")
    p.add_argument("--blocks", type=int, default=0,
                   help="also time K consecutive blocks of multi-block generation (each block generated, then "
                        "appended to the prefix by the context tower): reported under 'multiblock'")
    p.add_argument("--calibrate-copy-mb", type=int, default=0,
                   help="before the timed region, one device-to-device copy of this many MiB (a plain copy "
                        "kernel of known size, the scale of the HBM byte counters)")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="no benchmark: turn the counter CSVs of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; "
                        "both with --calibrate-copy-mb) into the LM head's HBM traffic record under profiles/")
    return p.parse_args()


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "block_diffusion_lm_step_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


LMHEAD_SOURCES = ("k_gemm.hip", "td_device.h", "td_kernels.h")
# Names of the LM-head kernels: activations staged in LDS (at most 16 rows, d <= 2048,
# the bench workload) and the row-list variant.
LMHEAD_KERNELS = ("lmhead_lds_kernel", "lmhead_kernel")


def lmhead_kernel_name(w) -> str:
    """The LM-head kernel the library plans for this workload's first step (all rows masked)."""
    M = w.n * w.B
    if w.dtype == "bf16" and M <= 16 and w.d <= 2048 and w.V % 512 == 0:
        k = "lmhead_lds_kernel (activations staged in LDS)"
    elif w.dtype == "bf16" and M >= 128 and w.V % 128 == 0 and w.d % 32 == 0:
        k = "gemm_tile_kernel<VSTAT> (128x128 MFMA tiles)"
    else:
        k = "lmhead_kernel (row-list gather)"
    return k + ": LM head GEMM + fused tau-scaled vocab max/sumexp/argmax"


def traffic_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"lmhead_{workload}_traffic.json")


def traffic_record(workload: str):
    """HBM bytes per LM-head launch from the rocprofv3 counters, if taken on the current source."""
    try:
        with open(traffic_path(workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != source_hash(*LMHEAD_SOURCES):
        return None
    return rec.get("hbm_bytes_per_launch")


def write_traffic(workload: str, fetch_csv: str, write_csv: str, calib_mb: int) -> dict:
    """Counter values per dispatch (KiB) -> bytes, scaled by the calibration copy.

    The copy of calib_mb MiB reads and writes exactly that many bytes; the ratio of that
    size to what FETCH_SIZE / WRITE_SIZE report for it scales the LM head's readings.
    LM-head dispatches that exited early (the block was already adopted) read ~nothing
    and are left out: the record is per working launch, like the bench's timing.
    """
    import csv

    def per_dispatch(path, counter):
        lm, blit, elem = [], [], []
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                v = float(row["Counter_Value"]) * 1024.0
                k = row["Kernel_Name"]
                if any(n in k for n in LMHEAD_KERNELS):
                    lm.append(v)
                elif "copyBuffer" in k:
                    blit.append(v)
                elif "MulFunctor" in k:
                    elem.append(v)
        return lm, blit, elem

    calib = calib_mb * 1024 * 1024
    out = {}
    for name, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        lm, blit, elem = per_dispatch(path, counter)
        if not lm or not elem:
            raise SystemExit(f"{path}: no LM-head or calibration dispatches with {counter}")
        factor = calib / max(elem)
        work = sorted(v for v in lm if v > 0.5 * max(lm)) if name == "fetch" else sorted(lm)
        if name == "fetch":
            fetch_work = len(work)
        raw = float(np.median(work))
        out[name] = dict(counter=counter, raw_bytes_per_launch=raw, calibration_kernel="elementwise (16 B per lane)",
                         calibration_raw_bytes=max(elem), factor=factor, bytes_per_launch=raw * factor,
                         dispatches=len(work), blit_copy_raw_bytes=max(blit) if blit else None)
    rec = dict(kernel="/".join(LMHEAD_KERNELS), workload=workload, source_sha256_16=source_hash(*LMHEAD_SOURCES),
               calibration_copy_bytes=calib, fetch=out["fetch"], write=out["write"],
               hbm_bytes_per_launch=out["fetch"]["bytes_per_launch"] + out["write"]["bytes_per_launch"],
               working_launches=fetch_work)
    os.makedirs(os.path.dirname(traffic_path(workload)), exist_ok=True)
    with open(traffic_path(workload), "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def cpu_baseline(w, budget_s: float):
    """The oracle as it stands, on this host's cores, on a bounded sample of the workload."""
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
    n_s = min(w.n, 4)   # sequences of the sample (all of a batch-1 workload)
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
        for s in range(n_s):
            kv(l, s)
        for name in ("wq", "wk", "wv", "wo", "attn_norm", "mlp_norm") + (() if w.moe else ("w1", "w2")):
            orc._w(name, l)
    for name in ("lm_head", "pos_emb", "final_norm"):
        orc._w(name)
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
    return dict(value=committed / dt, unit="committed tokens/s", cores=int(threads), kind="oracle", sample=sample,
                denoise_steps_per_s=steps / dt, seconds=dt)


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
                timing="host clock around K td_ar_step calls (each waits for the stream: the work lists are rebuilt "
                       "on the host)")


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
        t_gen = t_app = 0.0
        for _ in range(K):
            a = time.perf_counter()
            dev.generate_block(tok, com, tau, w.gamma, steps=steps)
            dev.sync()
            b = time.perf_counter()
            dev.append_block(tok)
            dev.sync()
            t_gen += b - a
            t_app += time.perf_counter() - b
        return t_gen, t_app

    run()
    reps = 3
    tg = ta = 0.0
    for _ in range(reps):
        g, a = run()
        tg += g
        ta += a
    tg, ta = tg / reps, ta / reps
    log(f"[bench] multi-block: {K} blocks, generate {tg * 1e3:.2f} ms, append {ta * 1e3:.2f} ms")
    return dict(blocks=K, value=round(K * w.n * w.B / (tg + ta), 3), unit="committed tokens/s",
                ms_per_block_generate=round(tg * 1e3 / K, 4), ms_per_block_append=round(ta * 1e3 / K, 4),
                timing="host clock around each call with a stream sync after it (the append rebuilds the "
                       "work lists on the host)")


def main():
    args = parse()
    if args.traffic_from:
        if args.calibrate_copy_mb <= 0:
            raise SystemExit("--traffic-from needs the --calibrate-copy-mb the counter runs used")
        print(json.dumps(write_traffic(args.workload, *args.traffic_from, args.calibrate_copy_mb)))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the library has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    from block_diffusion_lm_step_amd import (TD_PROF_ATTENTION, TD_PROF_GEMM, TD_PROF_LMHEAD, TD_PROF_MOE,
                                             TD_PROF_STEP, Denoiser)
    from synth import draw_inv_temp, draw_prefix_lengths, draw_tower, get_workload
    from synth.device import prefix_to_device, tower_config, tower_to_device

    w = get_workload(args.workload)
    if args.gamma is not None:
        w = w.with_(gamma=args.gamma)
    log(f"[bench] workload {w.name}: n={w.n} B={w.B} d={w.d} H={w.H}/{w.Hkv}x{w.hd} L={w.L} F={w.F} V={w.V} "
        f"gamma={w.gamma}")
    t = time.time()
    tw = draw_tower(w)
    dW = tower_to_device(tw)
    del tw
    plens = draw_prefix_lengths(w)
    offsets, ks, vs = prefix_to_device(w, plens)
    tau = torch.from_numpy(draw_inv_temp(w)).cuda()
    room = args.blocks * w.B * w.n   # tokens appended by --blocks
    dev = Denoiser(tower_config(w, max_batch=w.n, max_prefix_tokens=max(1, offsets[-1] + room)), dW)
    del dW
    if w.moe:   # every layer's MLP a mixture of experts
        from synth import draw_moe
        from synth.device import moe_config, moe_to_device
        dM = moe_to_device(draw_moe(w))
        dev.set_moe(moe_config(w), dM)
        del dM
    dev.set_prefix(offsets, ks, vs)
    if args.issue_window > 0:
        dev.set_issue_window(args.issue_window)
    torch.cuda.synchronize()
    log(f"[bench] inputs resident in HBM ({time.time() - t:.1f} s)")

    tok = torch.zeros((w.n, w.B), dtype=torch.int32, device="cuda")
    com = torch.zeros((w.n, w.B), dtype=torch.uint8, device="cuda")
    steps = torch.zeros(w.n, dtype=torch.int32, device="cuda")

    def block():
        dev.generate_block(tok, com, tau, w.gamma, steps=steps)

    for _ in range(args.warmup):
        block()
    dev.sync()
    if args.calibrate_copy_mb > 0:
        # Two copies of known size: the runtime's blit copy, and an elementwise kernel
        # whose lanes move 16 contiguous bytes each (1 KiB per wave instruction, the
        # access pattern of the weight streams).
        nb = args.calibrate_copy_mb * 1024 * 1024
        src = torch.ones(nb // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    log("[bench] warmup done")

    # The dominant kernel's launches are timed inside the timed region: the LM head, or
    # with a mixture of experts the expert projections.
    dev.profile_begin(TD_PROF_MOE if w.moe else TD_PROF_LMHEAD)
    if w.moe:
        dev.moe_stats()   # reset the expert counters
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        block()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    lm_ms = dev.profile_end()
    moe_launches, moe_active = dev.moe_stats() if w.moe else (0, 0)
    dev.sync()
    elapsed = t1 - t0
    st = steps.cpu().numpy()
    S = int(st.max())
    assert com.cpu().numpy().all(), "block not fully committed"
    log(f"[bench] {args.steps} blocks in {elapsed * 1e3:.2f} ms; steps per block {st.tolist()}")

    tokens_per_s = args.steps * w.n * w.B / elapsed
    steps_per_s = args.steps * S / elapsed
    elt = 2 if w.dtype == "bf16" else 4
    if w.moe:
        # Expert launches that did work: per working step, L layers x (up, down).  Each
        # reads the W1 (or W2) of every expert that holds a row, once: the counters give
        # the experts per layer-step.
        issued = len(lm_ms) // (args.steps * w.L * 2)   # steps issued per block (fewer than B with a window)
        assert issued * args.steps * w.L * 2 == len(lm_ms) and issued >= S, (len(lm_ms), args.steps, S)
        lm = np.array(lm_ms).reshape(args.steps, issued, w.L, 2)[:, :S]
        assert moe_launches == args.steps * S * w.L, (moe_launches, args.steps, S)
        active_per_layer = moe_active / moe_launches
        lm_bytes = int(round(active_per_layer * w.moe[3] * w.d * elt))
        kernel = ("moe_gemm_kernel: expert up (gathered rows, GELU) and down projections, weights of the "
                  f"{active_per_layer:.1f} experts (routed + shared) holding a row per layer")
        traffic = None
    else:
        # LM-head launches that did work: the first S of every block's launches (B, or
        # fewer with an issue window; every block is the same).
        issued = len(lm_ms) // args.steps
        assert issued * args.steps == len(lm_ms) and issued >= S, (len(lm_ms), args.steps, S)
        lm = np.array(lm_ms).reshape(args.steps, issued)[:, :S]
        lm_bytes = w.V * w.d * elt
        kernel = lmhead_kernel_name(w)
        traffic = traffic_record(w.name)
    lm_avg_ms = float(lm.mean())
    achieved = lm_bytes / (lm_avg_ms * 1e-3) / 1e9

    breakdown = {}
    if args.breakdown:
        kinds = (("gemm", TD_PROF_GEMM), ("attention", TD_PROF_ATTENTION), ("step", TD_PROF_STEP))
        if w.moe:
            kinds += (("moe_experts", TD_PROF_MOE),)
        dev.set_issue_window(0)   # B steps per block: launches per step are read off the record
        for name, kind in kinds:
            dev.profile_begin(kind)
            for _ in range(3):
                block()
            ms = np.array(dev.profile_end())
            per = len(ms) // (3 * w.B)
            ms = ms.reshape(3, w.B, per)[:, :S, :]
            breakdown[name] = dict(ms_per_step=float(ms.sum(axis=2).mean()), launches_per_step=per)
        dev.set_issue_window(args.issue_window)
        step_bytes = (w.weight_params(moe_active / max(1, moe_launches)) * elt
                      + int(plens.sum()) * w.L * 2 * w.Hkv * w.hd * elt)
        breakdown["step_alg_bytes"] = step_bytes
        breakdown["step_hbm_frac"] = step_bytes / (breakdown["step"]["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS

    multiblock = None
    if args.blocks > 0:
        multiblock = time_multiblock(args, w, plens, tau, dev, tok, com, steps)
    ar = None
    if args.ar > 0:
        ar = time_ar(args, w, plens)
        ar["diffusion_to_ar"] = round((multiblock["value"] if multiblock else tokens_per_s) / ar["value"], 4)

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 3),
        "unit": "committed tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; random-init tower weights N(0,0.02), prefix K/V N(0,1))",
        "config": {"workload": w.name, "batch": w.n, "prefix_tokens": int(plens.sum()), "block": w.B, "gamma": w.gamma,
                   "issue_window": args.issue_window,
                   "d_model": w.d, "heads": w.H, "kv_heads": w.Hkv, "head_dim": w.hd, "layers": w.L, "d_ff": w.F,
                   "vocab": w.V, **({"moe": {"experts": w.moe[0], "top_k": w.moe[1], "shared": w.moe[2],
                                              "d_expert": w.moe[3]}} if w.moe else {})},
        "denoise_steps_per_s": round(steps_per_s, 3),
        "denoise_steps_per_block": S,
        "roofline": {"kernel": kernel,
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "alg_bytes_per_launch": lm_bytes, "avg_launch_ms": round(lm_avg_ms, 5),
                     "launches_averaged": int(lm.size)},
    }
    if breakdown:
        out["breakdown"] = breakdown
    if multiblock:
        out["multiblock"] = multiblock
    if ar:
        out["ar"] = ar
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle sample")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    dev.close()


if __name__ == "__main__":
    main()
