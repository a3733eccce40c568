#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = the whole path once: the forward pass (O, L) and the backward pass
(D, the K/V-tile loop for dK/dV, the dQ pass) of causal bf16
attention, B=4, H=16, N=8192, d=128, on seeded synthetic N(0,1) inputs that
are resident in HBM before timing starts.

FLOPs follow the FlashAttention-2 convention (summary page, section 3
"FLOPs"): forward 4*B*H*N^2*d, halved with the causal mask; backward 2.5x
the forward.  Peak: MI355X dense bf16 matrix-core rate, 256 CUs x 2.4 GHz x
4096 FLOP/clk = 2516.6 TFLOP/s.

Prints ONE JSON line on stdout (progress goes to stderr).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
METRIC = "attention TFLOP/s fwd & bwd (bf16, d=128, causal) and % of MI355X MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_kv_kernel_b4_h16_n8192_d128_causal_hbm_traffic.json")
COPY_PROBE_BYTES = 512 << 20     # plain device copy timed by --probe to calibrate the HBM byte counters


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_traffic(launches_per_dispatch: float = 1.0):
    """HBM bytes per launch of the backward K/V-tile kernel from committed
    rocprofv3 counter runs, or None when absent or taken on a different
    kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    from exact_io_aware_26_amd.profiling import kernel_source_digest
    if t.get("source_sha256") != kernel_source_digest():
        return None
    return float(t["bytes_per_launch"]) * launches_per_dispatch


def _half_ulp_bf16(ref):
    import numpy as np
    a = np.maximum(np.abs(ref), 2.0 ** -126)
    return np.ldexp(1.0, (np.floor(np.log2(a)) - 8).astype(np.int64))


class _ParityAccumulator:
    """Errors of GPU outputs against the fp64 oracle over the sampled heads: raw max-abs,
    max-abs beyond the output's own bf16 rounding (half an ulp of the exact value), and
    relative L2 over all sampled elements."""

    def __init__(self):
        self.acc = {}

    def add(self, name, got, ref):
        import numpy as np
        err = np.abs(got - ref)
        a = self.acc.setdefault(name, {"max_abs": 0.0, "beyond": 0.0, "num": 0.0, "den": 0.0,
                                       "finite": True})
        a["max_abs"] = max(a["max_abs"], float(err.max()))
        a["beyond"] = max(a["beyond"], float(np.maximum(0.0, err - _half_ulp_bf16(ref)).max()))
        a["num"] += float(np.sum((got - ref) ** 2))
        a["den"] += float(np.sum(ref ** 2))
        a["finite"] = a["finite"] and bool(np.all(np.isfinite(got)))

    def report(self, gates):
        out, ok = {}, True
        for name, a in self.acc.items():
            r = {"max_abs": a["max_abs"], "finite": a["finite"]}
            if name == "L":
                ok = ok and a["finite"] and a["max_abs"] <= gates["L_max_abs"]
            else:
                r["max_abs_beyond_rounding"] = a["beyond"]
                r["rel_l2"] = (a["num"] / a["den"]) ** 0.5 if a["den"] > 0 else 0.0
                ok = ok and a["finite"] and r["max_abs_beyond_rounding"] <= gates["max_abs_beyond_rounding"] \
                    and r["rel_l2"] <= gates["rel_l2"]
            out[name] = r
        return out, ok


def cpu_baseline(w, qb, kb, vb, dob, budget_s: float, gpu_out=None):
    """The fp64 oracle on whole (batch, head) slices of the same inputs until ~budget_s.

    gpu_out: optional callable (b, hq) -> {"split_o": ..., "plain_o": ...}, each a dict of
    the GPU's outputs of that head as float64 arrays (the timed step's O, L, dQ and, with
    one query head per K/V head, dK, dV; the plain-O backward's dQ, dK, dV); the
    oracle's results of every timed slice are then compared with them (outside the
    timed region) and the errors returned as the second value."""
    import numpy as np
    from exact_io_aware_26_amd import inputs
    from oracle import oracle as orc

    lib = orc.load()
    G = w.Hq // w.Hkv
    heads, flops, t_total = 0, 0.0, 0.0
    per_head_flops = (w.fwd_flops() + w.bwd_flops()) / (w.B * w.Hq)
    par, par_plain = _ParityAccumulator(), _ParityAccumulator()
    while heads < w.B * w.Hq:
        b, hq = divmod(heads, w.Hq)
        hk = hq // G
        q = inputs.bf16_bits_to_f64(qb[b:b + 1, hq:hq + 1])
        k = inputs.bf16_bits_to_f64(kb[b:b + 1, hk:hk + 1])
        v = inputs.bf16_bits_to_f64(vb[b:b + 1, hk:hk + 1])
        do = inputs.bf16_bits_to_f64(dob[b:b + 1, hq:hq + 1])
        t0 = time.perf_counter()
        ro, rL = orc.forward(q, k, v, w.causal, w.scale, lib=lib)
        rdq, rdk, rdv, _ = orc.backward(q, k, v, do, w.causal, w.scale, lib=lib)
        t_total += time.perf_counter() - t0
        flops += per_head_flops
        heads += 1
        if gpu_out is not None:
            got = gpu_out(b, hq)
            ref = {"O": ro[0, 0], "L": rL[0, 0], "dQ": rdq[0, 0], "dK": rdk[0, 0], "dV": rdv[0, 0]}
            for name, x in got["split_o"].items():
                par.add(name, x, ref[name])
            for name, x in got["plain_o"].items():
                par_plain.add(name, x, ref[name])
        log(f"cpu baseline: {heads} head(s) in {t_total:.1f} s")
        if t_total >= budget_s:
            break
    cpu = {
        "value": flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": orc.num_threads(lib),
        "kind": "oracle",
        "sample": (f"fp64 oracle forward+backward of {heads} whole (batch, head) slice(s) "
                   f"[1,1,{w.N},{w.d}] causal of the same inputs, {t_total:.1f} s; "
                   "rate = the slices' FLOPs (same convention) / wall time"),
    }
    if gpu_out is None:
        return cpu, None
    gates = {"max_abs_beyond_rounding": 1e-2, "rel_l2": 5e-3, "L_max_abs": 1e-3}
    errors, ok = par.report(gates)
    parity = {"against": "fp64 oracle", "sample": f"the {heads} (batch, head) slice(s) timed above, "
              "outputs of the last timed step (split O: D from O + O_lo)", "gates": gates, "pass": ok,
              "errors": errors}
    if par_plain.acc:
        errors_plain, ok_plain = par_plain.report(gates)
        parity["plain_o"] = {"sample": "the same slices through fa2_bwd (D from the bf16 O alone)",
                             "pass": ok_plain, "errors": errors_plain}
    return cpu, parity


def _median_ms(torch, fn, warmup=20, groups=5, per_group=10):
    """Median and minimum over `groups` of the mean time per call of `per_group`
    back-to-back calls (events around each group, on the current stream), after
    `warmup` calls."""
    for _ in range(warmup):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(groups)]
    for a, b in ev:
        a.record()
        for _ in range(per_group):
            fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) / per_group for a, b in ev)
    return t[len(t) // 2], t[0]


def extra_figures(torch, fa2, workloads, dev):
    """Forward of every throughput configuration, and the backward at their shapes.

    Inputs are iid N(0,1) bf16 drawn on the device from each configuration's seed
    (the same distribution as the parity inputs; only the generator differs).
    """
    out = {}
    fwd_cfgs = (workloads.SHORT_NONCAUSAL, workloads.SHORT_CAUSAL, workloads.LONG,
                workloads.GQA_D128, workloads.GQA_D256)
    bwd_cfgs = (workloads.SHORT_NONCAUSAL, workloads.SHORT_CAUSAL, workloads.GQA_D128, workloads.GQA_D256)
    for wl in fwd_cfgs:
        log(f"extra figures: {wl.name}")
        g = torch.Generator(device=dev).manual_seed(wl.seed)
        mk = lambda h: torch.randn(wl.B, h, wl.N, wl.d, device=dev, dtype=torch.bfloat16, generator=g)
        q, k, v = mk(wl.Hq), mk(wl.Hkv), mk(wl.Hkv)
        o, lse = fa2.forward(q, k, v, causal=wl.causal)
        med, mn = _median_ms(torch, lambda: fa2.forward(q, k, v, causal=wl.causal, out=o, lse=lse))
        rec = {"fwd_ms": med, "fwd_ms_min": mn, "fwd_tflops": wl.fwd_flops() / (med * 1e-3) / 1e12}
        rec["fwd_pct_peak"] = 100 * rec["fwd_tflops"] / PEAK_BF16_TFLOPS
        if wl in bwd_cfgs:
            do = mk(wl.Hq)
            ws = torch.empty(fa2.workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.N, wl.d), dtype=torch.uint8, device=dev)
            grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
            med, mn = _median_ms(torch, lambda: fa2.backward(q, k, v, o, lse, do, causal=wl.causal,
                                                             workspace=ws, grads=grads))
            rec.update({"bwd_ms": med, "bwd_ms_min": mn, "bwd_tflops": wl.bwd_flops() / (med * 1e-3) / 1e12})
            rec["bwd_pct_peak"] = 100 * rec["bwd_tflops"] / PEAK_BF16_TFLOPS
            del do, ws, grads
        out[wl.name] = rec
        del q, k, v, o, lse
    # Block-sparse attention at the headline shape: a sliding window of 4 key
    # blocks plus key block 0 (causal), and a random quarter of the blocks
    # (non-causal).  FLOPs count only the kept blocks.
    from exact_io_aware_26_amd import inputs
    wl = workloads.BWD
    for kind, causal, d, name in (("local_global", True, 128, "block_sparse_local_global_causal_b4_h16_n8192_d128"),
                                  ("random", False, 128, "block_sparse_random25_b4_h16_n8192_d128"),
                                  ("random", False, 256, "block_sparse_random25_b4_h16_n8192_d256")):
        log(f"extra figures: {name}")
        mask_np = inputs.block_mask(kind, wl.N, seed=wl.seed, density=0.25)
        bm = torch.from_numpy(mask_np).to(dev)
        g = torch.Generator(device=dev).manual_seed(wl.seed)
        mk = lambda h: torch.randn(wl.B, h, wl.N, d, device=dev, dtype=torch.bfloat16, generator=g)
        q, k, v, do = mk(wl.Hq), mk(wl.Hkv), mk(wl.Hkv), mk(wl.Hq)
        o, lse = fa2.forward_block_sparse(q, k, v, bm, causal=causal)
        fmed, fmn = _median_ms(torch, lambda: fa2.forward_block_sparse(q, k, v, bm, causal=causal, out=o, lse=lse))
        ws = torch.empty(fa2.workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.N, d), dtype=torch.uint8, device=dev)
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        bmed, bmn = _median_ms(torch, lambda: fa2.backward_block_sparse(q, k, v, o, lse, do, bm, causal=causal,
                                                                        workspace=ws, grads=grads))
        ff = workloads.block_sparse_fwd_flops(mask_np, wl.B, wl.Hq, wl.N, d, causal)
        out[name] = {"kept_blocks": int(mask_np.sum()), "blocks": int(mask_np.size),
                     "fwd_ms": fmed, "fwd_ms_min": fmn, "fwd_tflops": ff / (fmed * 1e-3) / 1e12,
                     "bwd_ms": bmed, "bwd_ms_min": bmn, "bwd_tflops": 2.5 * ff / (bmed * 1e-3) / 1e12}
        del q, k, v, do, o, lse, ws, grads, bm
    # The headline shape's backward with the pages' atomic accumulation of dQ (the
    # FA2_BWD_DQ_ATOMIC mode: dQ added into an fp32 accumulator inside the K/V loop).
    wl = workloads.BWD
    log(f"extra figures: {wl.name} backward, atomic dQ")
    g = torch.Generator(device=dev).manual_seed(wl.seed)
    mk = lambda h: torch.randn(wl.B, h, wl.N, wl.d, device=dev, dtype=torch.bfloat16, generator=g)
    q, k, v, do = mk(wl.Hq), mk(wl.Hkv), mk(wl.Hkv), mk(wl.Hq)
    o, lse = fa2.forward(q, k, v, causal=wl.causal)
    mode = fa2.BWD_ALL | fa2.BWD_DQ_ATOMIC
    ws = torch.empty(fa2.workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.N, wl.d, stages=mode), dtype=torch.uint8,
                     device=dev)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    bmed, bmn = _median_ms(torch, lambda: fa2.backward(q, k, v, o, lse, do, causal=wl.causal, workspace=ws,
                                                       grads=grads, stages=mode), warmup=5, groups=3, per_group=5)
    out[wl.name + "_bwd_atomic_dq"] = {"bwd_ms": bmed, "bwd_ms_min": bmn,
                                       "bwd_tflops": wl.bwd_flops() / (bmed * 1e-3) / 1e12}
    del q, k, v, do, o, lse, ws, grads
    # The headline shape with f16 inputs and outputs (the fa2_*_f16 entry points).
    wl = workloads.BWD
    log(f"extra figures: {wl.name} in f16")
    g = torch.Generator(device=dev).manual_seed(wl.seed)
    mk = lambda h: torch.randn(wl.B, h, wl.N, wl.d, device=dev, dtype=torch.float16, generator=g)
    q, k, v, do = mk(wl.Hq), mk(wl.Hkv), mk(wl.Hkv), mk(wl.Hq)
    o, lse = fa2.forward(q, k, v, causal=wl.causal)
    fmed, _ = _median_ms(torch, lambda: fa2.forward(q, k, v, causal=wl.causal, out=o, lse=lse))
    ws = torch.empty(fa2.workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.N, wl.d), dtype=torch.uint8, device=dev)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    bmed, _ = _median_ms(torch, lambda: fa2.backward(q, k, v, o, lse, do, causal=wl.causal, workspace=ws,
                                                     grads=grads), warmup=5, groups=3, per_group=5)
    out[wl.name + "_f16"] = {"fwd_ms": fmed, "fwd_tflops": wl.fwd_flops() / (fmed * 1e-3) / 1e12,
                             "bwd_ms": bmed, "bwd_tflops": wl.bwd_flops() / (bmed * 1e-3) / 1e12}
    return out

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline (0 to skip)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other configurations' figures and the plain-O comparison")
    ap.add_argument("--probe", action="store_true",
                    help="for profilers: one plain copy of known size, then one forward and each backward "
                         "stage once; prints no JSON")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path, so --gpus {args.gpus} "
              "is not supported; run with --gpus 1", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch

    from exact_io_aware_26_amd import fa2, inputs, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    fa2.load()
    dev = torch.device("cuda:0")
    w = workloads.BWD
    log(f"workload {w.name}: generating seeded inputs")
    qb, kb, vb, dob = inputs.attention_inputs(w.seed, w.B, w.Hq, w.Hkv, w.N, w.d, with_grad=True)

    def to_dev(x):
        return torch.from_numpy(x.view("int16")).view(torch.bfloat16).to(dev)

    q, k, v, do = (to_dev(x) for x in (qb, kb, vb, dob))
    o = torch.empty_like(q)
    o_lo = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa2.workspace_bytes(w.B, w.Hq, w.Hkv, w.N, w.d), dtype=torch.uint8, device=dev)
    grads = (dq, dk, dv)

    # The step: the forward with O's rounding residual (fa2_fwd_olo) and the
    # backward forming D from O + O_lo (fa2_bwd_stages_olo).
    def fwd():
        fa2.forward(q, k, v, causal=w.causal, out=o, lse=lse, o_lo=o_lo)

    def bwd(stages):
        fa2.backward(q, k, v, o, lse, do, causal=w.causal, workspace=ws, grads=grads, stages=stages,
                     o_lo=o_lo)

    if args.probe:
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)                     # reads and writes COPY_PROBE_BYTES each
        torch.cuda.synchronize()
        del src, dst
        fwd()
        for stages in (fa2.BWD_PREPROCESS, fa2.BWD_MAIN, fa2.BWD_FINALIZE):
            bwd(stages)
        torch.cuda.synchronize()
        log("probe done")
        return 0

    log(f"warmup {args.warmup} step(s)")
    for _ in range(args.warmup):
        fwd()
        bwd(fa2.BWD_ALL)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    log(f"timing {args.steps} step(s)")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        e = ev[s]
        e[0].record()
        fwd()
        e[1].record()
        bwd(fa2.BWD_PREPROCESS)
        e[2].record()
        bwd(fa2.BWD_MAIN)
        e[3].record()
        bwd(fa2.BWD_FINALIZE)
        e[4].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_per_step = wall_ms / args.steps

    def avg(i, j):
        return sum(e[i].elapsed_time(e[j]) for e in ev) / args.steps

    fwd_ms, pre_ms, main_ms, dq_ms = avg(0, 1), avg(1, 2), avg(2, 3), avg(3, 4)
    bwd_ms = pre_ms + main_ms + dq_ms
    fwd_f, bwd_f = w.fwd_flops(), w.bwd_flops()
    value = (fwd_f + bwd_f) / (ms_per_step * 1e-3) / 1e12
    log(f"step {ms_per_step:.3f} ms: fwd {fwd_ms:.3f} ms, bwd D {pre_ms:.3f} + dK/dV loop {main_ms:.3f} "
        f"+ dQ pass {dq_ms:.3f} ms")

    # The dominant kernel is the backward K/V-tile loop (bwd_kv_kernel).  Its
    # algorithmic work is 4 of the backward's 5 products (S, dP, dV, dK), i.e.
    # 4/5 of the backward FLOPs; the dQ pass does the fifth (plus its recompute).
    main_flops = 0.8 * bwd_f
    main_tflops = main_flops / (main_ms * 1e-3) / 1e12
    traffic = measured_traffic()
    roofline = {
        "kernel": "bwd_kv_kernel<128, causal> (backward K/V-tile loop: S, dP, dV, dK)",
        "bound": "mfma",
        "achieved": main_tflops,
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": main_tflops / PEAK_BF16_TFLOPS,
        "traffic": traffic,
        "avg_launch_ms": main_ms,
        "algorithmic_flops_per_launch": main_flops,
    }

    extra = {}
    grads_plain = None
    if not args.no_extra:
        # The same step without the residual (fa2_fwd, fa2_bwd: D from the bf16 O),
        # timed as the extra figures are, its outputs kept for the parity record.
        log("plain-O step: fa2_fwd and fa2_bwd")
        grads_plain = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        pf_med, _ = _median_ms(torch, lambda: fa2.forward(q, k, v, causal=w.causal, out=o, lse=lse),
                               warmup=5, groups=3, per_group=10)
        pb_med, _ = _median_ms(torch, lambda: fa2.backward(q, k, v, o, lse, do, causal=w.causal, workspace=ws,
                                                           grads=grads_plain), warmup=5, groups=3, per_group=5)
        sf_med, _ = _median_ms(torch, fwd, warmup=5, groups=3, per_group=10)
        sb_med, _ = _median_ms(torch, lambda: bwd(fa2.BWD_ALL), warmup=5, groups=3, per_group=5)
        torch.cuda.synchronize()
        extra = extra_figures(torch, fa2, workloads, dev)
        extra[w.name + "_plain_o"] = {"fwd_ms": pf_med, "fwd_tflops": fwd_f / (pf_med * 1e-3) / 1e12,
                                      "bwd_ms": pb_med, "bwd_tflops": bwd_f / (pb_med * 1e-3) / 1e12,
                                      "split_o_fwd_ms": sf_med, "split_o_bwd_ms": sb_med}

    cpu, parity = None, None
    if args.cpu_budget > 0:
        log("cpu baseline (oracle) and parity of the timed step's outputs")
        G = w.Hq // w.Hkv

        def gpu_out(b, hq):
            def f64(t):
                return inputs.bf16_bits_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view("uint16"))
            out = {"O": f64(o[b, hq]), "L": lse[b, hq].double().cpu().numpy(), "dQ": f64(dq[b, hq])}
            if G == 1:
                out.update({"dK": f64(dk[b, hq]), "dV": f64(dv[b, hq])})
            plain_out = {}
            if grads_plain is not None:
                plain_out = {"dQ": f64(grads_plain[0][b, hq])}
                if G == 1:
                    plain_out.update({"dK": f64(grads_plain[1][b, hq]), "dV": f64(grads_plain[2][b, hq])})
            return {"split_o": out, "plain_o": plain_out}

        cpu, parity = cpu_baseline(w, qb, kb, vb, dob, args.cpu_budget, gpu_out)

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "causal": w.causal, "scale": w.scale, "seed": w.seed,
                   "entry_points": "fa2_fwd_olo + fa2_bwd_stages_olo (split O)"},
        "pct_of_peak": 100 * value / PEAK_BF16_TFLOPS,
        "fwd_ms": fwd_ms,
        "fwd_tflops": fwd_f / (fwd_ms * 1e-3) / 1e12,
        "bwd_ms": bwd_ms,
        "bwd_tflops": bwd_f / (bwd_ms * 1e-3) / 1e12,
        "bwd_stage_ms": {"preprocess_D": pre_ms, "dk_dv_loop": main_ms, "dq_pass": dq_ms},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
