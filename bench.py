"""Benchmark: draft + verify cycles/s and tokens/s of the one-pass block-
diffusion drafter on one MI355X.

A step is one full cycle (inject_kv -> block_draft -> lm_head_argmax ->
verify) over the batch of the workload, on synthetic inputs already resident
in HBM.  Default workload: the 8B-shaped drafter (5 layers, hidden 4096,
32/8 heads x 128, MLP 12288, vocabulary 151936) at batch 32 with ragged
contexts U[1024, 8192], block 16, temperature-1 rejection-sampling verify
with bf16 target logits N(0, 3) and Philox uniforms.

Prints ONE JSON line (see the keys at the end of main()).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
# Per-position acceptance of the planted variant: with gamma = 15 it gives
# E[tau] = 1 + sum_{j=1..15} 0.86^j = 6.50, the mean acceptance length the
# DFlash review's main results table (temperature 0) reports for the
# Qwen3-8B drafter with block size 16 (6.49).  Random weights alone give
# tau ~ 1.1.
PLANT_ALPHA = 0.86
MFMA_F32_PEAK_TFLOPS = 157.3


def _algorithmic(cfg, rows, n_inj):
    """Algorithmic bytes / flops of each library call for one cycle (weights
    and context K/V read once, activations, logits only where stored)."""
    d, V, L = cfg["hidden"], cfg["vocab"], cfg["n_layers"]
    hq, hkv, dh, m = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["mlp"]
    F = cfg["feat_dim"]
    eb = 2 if cfg["dtype"] == "bf16" else 4
    bs, C, B, g = cfg["bs"], cfg["n_copies"], cfg["block"], cfg["gamma"]
    R = bs * C * B
    layer_params = (hq + 2 * hkv) * dh * d + d * hq * dh + 2 * m * d + d * m
    ctx = cfg["ctx_lens"]
    W, full = int(cfg.get("swa_window", 0)), int(cfg.get("full_attn_mask", 0))
    # context keys each layer reads: the last W under a sliding window
    seen = [[min(S, W) if W > 0 and not (full >> l) & 1 else S for S in ctx] for l in range(L)]
    attn_bytes = sum((S + B * C) * hkv * dh * 2 * eb for sl in seen for S in sl)
    attn_flops = sum(C * 4 * B * hq * dh * (S + B) for sl in seen for S in sl)
    head_logits = 4 * rows * V if cfg["verify"] == "rs" else 0
    head_bytes = eb * V * d + rows * (eb * d + 16) + head_logits
    head_flops = 2 * rows * V * d
    inj_params = d * F + 2 * hkv * dh * d * L
    inj_bytes = eb * inj_params + n_inj * (F * eb + L * 2 * hkv * dh * eb)
    inj_flops = 2 * n_inj * inj_params
    tsz = 2 if cfg.get("target_dtype") == "bf16" else 4
    ver_bytes = bs * (g + 1) * V * tsz + (bs * V * 4 if cfg["verify"] == "rs" else 0)
    if cfg["verify"] == "none":
        ver_bytes = 0
    if cfg["verify"] == "spot":  # per-slot head outputs and states of every copy
        ver_bytes = bs * C * B * 5 * 4
    draft_bytes = eb * L * layer_params + attn_bytes
    draft_flops = 2 * R * L * layer_params + attn_flops
    return dict(
        inject=dict(bytes=inj_bytes, flops=inj_flops),
        draft=dict(bytes=draft_bytes, flops=draft_flops, attn_bytes=attn_bytes,
                   attn_flops=attn_flops, gemm_bytes=eb * L * layer_params,
                   gemm_flops=2 * R * L * layer_params),
        head=dict(bytes=head_bytes, flops=head_flops),
        verify=dict(bytes=ver_bytes, flops=0),
    )


def _profiled_traffic(workload, kernel, files):
    """HBM bytes per dispatch of `kernel` from the committed rocprofv3 counter
    summary of `workload` (FETCH_SIZE and WRITE_SIZE scaled by a plain copy of
    known size), or None when there is none or the kernel's sources changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if line.startswith(f"[{kernel}] ") and ":" in line:
            k, v = line[len(kernel) + 3:].split(":", 1)
            vals[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "block_diffusion_speculative_kv_amd", "csrc", f), "rb").read())
    if vals.get("source_sha256_16") != h.hexdigest()[:16]:
        return None
    return int(float(vals["traffic_bytes_per_dispatch"]))


def _cpu_baseline(cfg, cyc, budget_s):
    """Time the CPU oracle on a bounded sample of the same workload: whole
    cycles for as many sequences as fit in ~budget_s, scaled to the batch,
    then again with BLAS held to one thread for a per-core figure."""
    import numpy as np

    from block_diffusion_speculative_kv_amd import KVCache
    from oracle.drafter import Drafter as OracleDrafter, lm_head
    from oracle import philox
    from oracle.verify import verify_batch

    def host(t):
        return t.detach().cpu().double().numpy()

    w = {k: (host(v) if not isinstance(v, list) else
             [{a: host(b) for a, b in l.items()} for l in v]) for k, v in cyc.w.items()}
    od = OracleDrafter(cfg, w)
    feats = host(cyc.feats)
    tokens = cyc.tokens.cpu().numpy()
    target = host(cyc.target) if cyc.verify_mode is not None else None
    n_new, g, V = cyc.n_new, cfg["gamma"], cfg["vocab"]
    T = float(cfg.get("temperature", 1.0))
    def one_cycle(b, S):
        """one sequence's full cycle on the oracle; returns its seconds"""
        ck = [host(k[b]) for k in cyc.kv.k]
        cv = [host(KVCache.untile_v(v[b:b + 1])[0]) for v in cyc.kv.v]   # -> [h, pos, dh]
        t0 = time.perf_counter()
        ks, vs = od.inject_rows(feats[b * n_new:(b + 1) * n_new], np.arange(S - n_new, S))
        for l in range(cfg["n_layers"]):
            ck[l][:, S - n_new:S] = ks[l].transpose(1, 0, 2)
            cv[l][:, S - n_new:S] = vs[l].transpose(1, 0, 2)
        hid = od.draft(ck, cv, tokens[b], S)
        if cyc.mode == 0:
            out = lm_head(w["lm_head"], hid[0, 1:], keep_logits=True)
        else:
            gm = np.stack([philox.gumbel_row(cyc.seed, 0, b, k, 0, V) for k in range(g)])
            out = lm_head(w["lm_head"], hid[0, 1:], temperature=T, gumbel=gm, keep_logits=True)
        if target is not None:
            mode = "rs" if cfg["verify"] == "rs" else "greedy"
            verify_batch(mode, target[b:b + 1], out["ids"][None, :],
                         zd=out["logits"][None, :], temperature=T, seed=cyc.seed, cycle=0)
        return time.perf_counter() - t0

    done, t_total = 0, 0.0
    for b, S in enumerate(cfg["ctx_lens"]):
        t_total += one_cycle(b, S)
        done += 1
        if t_total >= budget_s:
            break
    per_seq = t_total / done
    cycles_per_s = 1.0 / (per_seq * cfg["bs"])
    # the same oracle with its BLAS held to one thread, on the first
    # sequences (a per-core figure; about a third of the budget)
    single = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas = sorted({f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info()
                       if i.get("user_api") == "blas"})
        with threadpool_limits(1):
            d1, t1 = 0, 0.0
            for b, S in enumerate(cfg["ctx_lens"]):
                t1 += one_cycle(b, S)
                d1 += 1
                if t1 >= budget_s / 3:
                    break
        single = dict(value=1.0 / (t1 / d1 * cfg["bs"]), unit="cycles/s", cores=1,
                      sample=f"{d1} of {cfg['bs']} sequences ({t1:.1f} s), BLAS held to one thread")
    except ImportError:  # pragma: no cover
        blas = []
    cpu_model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    return dict(value=cycles_per_s, unit="cycles/s", cores=len(os.sched_getaffinity(0)),
                kind="oracle",
                sample=f"{done} of {cfg['bs']} sequences, one full cycle each "
                       f"({t_total:.1f} s), scaled linearly to the batch",
                single_thread=single, cpu_model=cpu_model, blas=blas)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="q8b_bs32_rs")
    ap.add_argument("--n-new", type=int, default=8)
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--copy-mib", type=int, default=1024,
                    help="size of the calibration copy for HBM byte counters (0 = skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): the path shards "
              "over sequences with no per-cycle exchange, so the measure is one GPU's share "
              "at its real shape; no multi-GPU run is implemented", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_diffusion_speculative_kv_amd import _lib
    from block_diffusion_speculative_kv_amd.cycle import Cycle
    from synth import configs

    _lib.load()
    cfg = configs.get(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] workload {args.workload}: setting up (weights, prefill inject)", file=sys.stderr,
          flush=True)
    cyc = Cycle(cfg, device=dev, n_new=args.n_new)
    st = torch.cuda.current_stream()

    for i in range(args.warmup):
        cyc.step(cycle=i)
    torch.cuda.synchronize()

    # whole-cycle timing
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    taus = []
    ev0.record(st)
    for i in range(args.steps):
        cyc.step(cycle=args.warmup + i)
    ev1.record(st)
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps
    if cyc.yields:
        taus = cyc.tau.cpu().numpy().tolist()

    # per-call timing (same stream, events around each library call)
    if cyc.RK:
        names = ["inject", "refine", "verify"]
    else:
        names = ["inject", "draft", "head"] + (["loop"] if cyc.K else []) + ["verify"]
    evs = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)] for n in names}
    tau_hist = []
    for i in range(args.steps):
        c = args.warmup + args.steps + i
        calls = {"inject": cyc.inject, "draft": cyc.draft, "head": lambda: cyc.head(c),
                 "loop": lambda: cyc.loop(c), "verify": lambda: cyc.verify(c),
                 "refine": lambda: cyc.refine(c)}
        for n in names:
            fn = calls[n]
            evs[n][i][0].record(st)
            fn()
            evs[n][i][1].record(st)
        if cyc.yields and i < 8:
            tau_hist.append(cyc.tau.clone())
    torch.cuda.synchronize()
    per_call = {n: float(np.mean([a.elapsed_time(b) for a, b in evs[n]])) for n in names}
    if tau_hist:
        taus = torch.cat(tau_hist).cpu().numpy().tolist()
    tau_mean = float(np.mean(taus)) if taus else None

    # per-cycle spread: events between consecutive cycles, no host sync inside
    cev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    cev[0].record(st)
    for i in range(args.steps):
        cyc.step(cycle=args.warmup + 2 * args.steps + i)
        cev[i + 1].record(st)
    torch.cuda.synchronize()
    cyc_ms = np.array([cev[i].elapsed_time(cev[i + 1]) for i in range(args.steps)])
    cycle_ms = {q: round(float(np.percentile(cyc_ms, v)), 4)
                for q, v in (("p10", 10), ("median", 50), ("p90", 90))}

    # planted acceptance (plain one-pass cycles with verification): the same
    # cycles with accepted-prefix lengths planted into the target rows between
    # head and verification (harness work, untimed); the verification must
    # return tau = k + 1 for every sequence
    planted = None
    if cyc.can_plant():
        p_tau, p_bad = [], 0
        for i in range(args.steps):
            c = args.warmup + 3 * args.steps + i
            k = cyc.plant_draw(c, PLANT_ALPHA)
            cyc.step(cycle=c, plant_k=k)
            t = cyc.tau.cpu().numpy()
            p_bad += int(np.sum(t != k + 1))
            p_tau.append(t)
        planted = dict(alpha=PLANT_ALPHA, tau_mean=round(float(np.mean(p_tau)), 4),
                       tau_expected=round(1 + sum(PLANT_ALPHA ** j
                                                  for j in range(1, cyc.gamma + 1)), 4),
                       tau_mismatches=p_bad)

    n_inj = cfg["bs"] * cyc.n_new
    alg = _algorithmic(cfg, cyc.rows, n_inj)
    if cyc.K:
        # second pass: the drafter over K copies and the head over K gamma
        # rows; the joint verification reads every branch's target rows
        alg2 = _algorithmic(dict(cfg, n_copies=cyc.K), cyc.rows2, n_inj)
        alg["loop"] = dict(bytes=alg2["draft"]["bytes"] + alg2["head"]["bytes"],
                           flops=alg2["draft"]["flops"] + alg2["head"]["flops"])
        alg["verify"] = dict(bytes=alg["verify"]["bytes"] * cyc.K, flops=0)
    if cyc.RK:
        # K passes of the drafter and the head
        alg["refine"] = dict(bytes=cyc.RK * (alg["draft"]["bytes"] + alg["head"]["bytes"]),
                             flops=cyc.RK * (alg["draft"]["flops"] + alg["head"]["flops"]))
    cycles_per_s = 1000.0 / ms_step
    bs = cfg["bs"]
    tokens_per_s = cycles_per_s * bs * tau_mean if tau_mean else None
    if planted:
        # the cycle's work does not depend on tau (n_new is fixed), so the
        # planted tokens/s uses the timed cycle rate
        planted["tokens_per_s"] = round(cycles_per_s * bs * planted["tau_mean"], 1)
    total_bytes = sum(alg[n]["bytes"] for n in names)
    hbm_gbs = total_bytes / (ms_step * 1e-3) / 1e9

    # roofline of the LM-head call (one main kernel plus a small merge); in
    # the refinement rollout the head runs inside each pass and is timed once
    # on its own here
    if "head" not in per_call:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for i in range(args.steps):
            cyc.head(0)
        e1.record(st)
        torch.cuda.synchronize()
        per_call["head"] = e0.elapsed_time(e1) / args.steps
    head_s = per_call["head"] * 1e-3
    head_bound = "mfma" if alg["head"]["flops"] / alg["head"]["bytes"] > \
        MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9) else "hbm"
    # the LM-head kernel that runs at this row count (see launch_lm_head)
    if cfg["dtype"] != "bf16":
        head_kernel = "lm_head_kernel<float>"
    else:
        # mirrors launch_lm_head: the weight-streaming kernel up to 160 rows
        # (128-deep stages up to 64 rows, 64-deep beyond, when they divide the
        # depth), the tile engine otherwise
        r, d = cyc.rows, cfg["hidden"]
        rt = (r + 15) // 16
        ks = 128 if rt <= 4 else 64
        if r <= 160 and d % ks == 0:
            head_kernel = "lm_head_stream_kernel (%d row tiles, %d-deep stages)" % (
                rt if rt <= 4 else rt + (rt & 1), ks)
        else:
            head_kernel = "lm_head_lds_kernel (%d ids x %d rows tile)" % (
                (64, 32) if r <= 32 else (64, 64) if r <= 64
                else (128, 160) if r <= 160 else (256, 256))
    head_kernel += " (+lm_combine_kernel)"
    traffic = None
    if cfg["dtype"] == "bf16":
        traffic = _profiled_traffic(args.workload, head_kernel.split(" ")[0],
                                    ["lm_head.hip", "mma_tile.hpp", "dma.hpp", "common.hpp",
                                     "kernels.hpp"])
    if head_bound == "mfma":
        ach = alg["head"]["flops"] / head_s / 1e12
        roof = dict(kernel=head_kernel, bound="mfma", achieved=round(ach, 2),
                    peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s", frac=round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                    traffic=traffic, avg_us=round(per_call["head"] * 1e3, 2))
    else:
        ach = alg["head"]["bytes"] / head_s / 1e9
        roof = dict(kernel=head_kernel, bound="hbm", achieved=round(ach, 1),
                    peak=HBM_PEAK_GBS, unit="GB/s", frac=round(ach / HBM_PEAK_GBS, 4),
                    traffic=traffic, avg_us=round(per_call["head"] * 1e3, 2))

    stages = {}
    for n in names:
        t = per_call[n] * 1e-3
        b, f = alg[n]["bytes"], alg[n]["flops"]
        stages[n] = dict(ms=round(per_call[n], 4), gbs=round(b / t / 1e9, 1) if t else None,
                         tflops=round(f / t / 1e12, 2) if t else None)

    # prefill-size injection (outside the cycle timing): one inject_kv call on
    # the first prefill chunk (8192 rows), algorithmic flops 2 rows (W_c + the
    # K/V rows of every layer) against the bf16 MFMA peak
    prefill = None
    if cfg["dtype"] == "bf16" and sum(cfg["ctx_lens"]) >= 8192:
        f, sq, ps = cyc.prefill_chunk(8192)
        n = f.shape[0]
        cyc.dr.inject_kv(f, sq, ps, cyc.kv, cyc.ws)
        torch.cuda.synchronize()
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        p0.record(st)
        for _ in range(reps):
            cyc.dr.inject_kv(f, sq, ps, cyc.kv, cyc.ws)
        p1.record(st)
        torch.cuda.synchronize()
        t = p0.elapsed_time(p1) / reps * 1e-3
        d, L, kvd = cfg["hidden"], cfg["n_layers"], cfg["n_kv_heads"] * cfg["head_dim"]
        fl = 2.0 * n * (d * cfg["feat_dim"] + L * 2 * kvd * d)
        prefill = dict(rows=n, ms=round(t * 1e3, 4), tflops=round(fl / t / 1e12, 1),
                       mfma_frac=round(fl / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4))
        del f, sq, ps

    # calibration copy of known size for HBM byte counters (outside timing):
    # one elementwise kernel that reads and writes `copy_mib` MiB
    copy_info = None
    if args.copy_mib > 0:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(st)
        torch.mul(src, 1.0, out=dst)
        c1.record(st)
        torch.cuda.synchronize()
        t = c0.elapsed_time(c1) * 1e-3
        copy_info = dict(kernel="torch mul-by-1 (elementwise copy)", read_bytes=n * 4,
                         write_bytes=n * 4, gbs=round(2 * n * 4 / t / 1e9, 1))
        del src, dst

    cpu = None
    # the oracle baseline times the one-pass cycle (inject, draft, head, greedy
    # or RS verify); workloads with a second pass, refinement passes or the
    # multi-copy layout are not that cycle, so they carry no baseline
    plain = not (cyc.K or cyc.RK or cyc.spot or cyc.mode == 2)
    if args.cpu_budget > 0 and plain:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        cpu = _cpu_baseline(cfg, cyc, args.cpu_budget)

    out = {
        "metric": "draft+verify cycles/s (bs=32, 8B-shaped drafter)" if args.workload == "q8b_bs32_rs"
        else f"draft+verify cycles/s ({args.workload})",
        "value": round(cycles_per_s, 3),
        "unit": "cycles/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": bs, "block": cfg["block"],
                   "gamma": cfg["gamma"], "ctx": cfg["ctx"] if isinstance(cfg["ctx"], str)
                   else cfg["ctx_lens"], "verify": cfg["verify"], "head": cfg["lm_mode"],
                   "n_new_per_cycle": cyc.n_new, **({"dloop_k": cyc.K} if cyc.K else {}),
                   **({"refine_k": cyc.RK} if cyc.RK else {}),
                   **({"swa_window": cfg["swa_window"]} if cfg.get("swa_window") else {})},
        "tokens_per_s": round(tokens_per_s, 1) if tokens_per_s else None,
        "tau_mean": tau_mean,
        "planted": planted,
        "cycle_ms": cycle_ms,
        "hbm_gbs": round(hbm_gbs, 1),
        "stages": stages,
        "roofline": roof,
        "cpu_baseline": cpu,
        "prefill_inject": prefill,
        "calibration_copy": copy_info,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
