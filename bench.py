"""Benchmark: attention tokens/s at 256K context on one MI355X.

One step = the whole hot path over one batch of seeded synthetic input:
  * prefill pair at T = 262,144 (B = 1, Hq = 32, Hkv = 8, d = 128, bf16): one gated-SWA
    layer (W = 128) and one full-causal global layer over the same Q/K/V;
  * one decode step for B = 32 sequences at context 262,144: a global layer over a full
    [32, 8, 262144, 128] cache and a gated-SWA layer over a 128-entry ring.
value = (prefill tokens + decode tokens) / step time, inputs resident in HBM.

Prints ONE JSON line (rank 0). Per-kernel times come from HIP events recorded on the
stream the library launches on (torch's current stream).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="approximate CPU time budget of the oracle sample")
    ap.add_argument("--workload", choices=["c4", "c2"], default="c4",
                    help="prefill shape of --only: c4 = B=1 T=262144 (default), c2 = B=4 T=4096")
    ap.add_argument("--only", choices=["swa_prefill", "global_prefill", "global_decode",
                                       "swa_decode", "copy"], default=None,
                    help="run just this call (warmup + steps launches, for profilers); "
                         "'copy' is a plain 1 GiB device copy used to calibrate counters")
    ap.add_argument("--model-decode", action="store_true",
                    help="decode step of the whole 32-layer hybrid stack (27 SWA rings + 5 "
                         "global caches, B=32 at context 262144): one batched call against "
                         "32 single-layer calls")
    ap.add_argument("--varlen", action="store_true",
                    help="packed-document prefill: 262144 tokens in 16 documents of 16K and "
                         "in 24 documents of mixed length (one JSON line per packing)")
    ap.add_argument("--backward", action="store_true",
                    help="backward pass of one SWA and one global layer at B=1, T=65536 "
                         "(the 32-layer stack's per-layer size)")
    ap.add_argument("--sweep", action="store_true",
                    help="attention-stack sweep: 32-layer hybrid / SWA 3:1 / full-attention "
                         "stacks at T = 4K .. 256K (one JSON line per T)")
    ap.add_argument("--configs", action="store_true",
                    help="every configuration of the measurement table (C1-C5) with the "
                         "per-call protocol: 5 warm-ups, median/min/p90 of >= 20 calls "
                         "(>= 5 for the 256K global layer and the stack), caches flushed "
                         "before each call; one JSON line per configuration and layer")
    ap.add_argument("--flush", choices=["read", "write"], default="read",
                    help="with --configs: evict the caches before each call by reading a 1 GiB "
                         "buffer (default) or by writing one; a written buffer leaves the "
                         "memory-side cache full of dirty lines whose write-back then shares "
                         "HBM with the measured call")
    ap.add_argument("--fused-k", action="store_true",
                    help="with --only global_prefill: no workspace, the K transform fused into "
                         "every K-tile load (the alternative to the K~ pre-pass)")
    ap.add_argument("--sweep-t", default="",
                    help="comma-separated sequence lengths for --sweep (default: all)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "global_prefill_T262144_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "global_attention_qk_amd", "csrc", f)
                  for f in ("prefill_bf16.hip", "common.h")]


def measured_traffic():
    """HBM bytes per launch of the global prefill attention kernel, from the committed
    counter summary (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter's reading
    for a plain copy of known size); None when the kernel source changed since."""
    import hashlib
    try:
        kv = {}
        for line in open(TRAFFIC_FILE):
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
        src = hashlib.sha256(b"".join(open(f, "rb").read() for f in KERNEL_SOURCES)).hexdigest()
        if kv.get("kernel_source_sha256") != src:
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


class ClockSampler:
    """The GPU's current shader clock (amdsmi, MHz), sampled about every 20 ms by a thread
    while the timed steps run. Reports nothing when amdsmi cannot be used."""

    def __init__(self):
        import threading
        self.samples, self.error = [], None
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            try:
                handles = amdsmi.amdsmi_get_processor_handles()
                h = handles[0]
                while not self._stop.is_set():
                    self.samples.append(
                        amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.SYS)["clk"])
                    self._stop.wait(0.02)
            finally:
                amdsmi.amdsmi_shut_down()
        except Exception as e:  # no amdsmi, no permission: no clock in the report
            self.error = f"{type(e).__name__}: {e}"

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join(timeout=5)

    def report(self):
        xs = [x for x in self.samples if isinstance(x, (int, float)) and x > 0]
        if not xs:
            return {"source": "amdsmi", "error": self.error or "no samples"}
        ys = sorted(xs)
        return {"source": "amdsmi current GFX clock during the timed steps (median: the "
                          "sustained clock; idle gaps between calls give the low samples)",
                "median_MHz": ys[len(ys) // 2], "mean_MHz": sum(xs) / len(xs),
                "min_MHz": ys[0], "max_MHz": ys[-1], "samples": len(xs)}


def measured_peaks():
    """What this GPU sustains on plain library work, next to the spec peaks: a 1 GiB
    device-to-device copy (read + write bytes / time) and a bf16 8192^3 matrix product
    (torch / hipBLASLt), each the best of 10 timed runs after warm-up."""
    import torch
    out = {}

    def best(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        return min(ts)

    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    x.fill_(3)
    out["hbm_copy_GBs"] = 2 * n / best(lambda: y.copy_(x)) / 1e9
    del x, y
    m = 8192
    a = torch.randn(m, m, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(m, m, device="cuda", dtype=torch.bfloat16)
    c = torch.empty(m, m, device="cuda", dtype=torch.bfloat16)
    out["bf16_gemm_TFLOPs"] = 2 * m ** 3 / best(lambda: torch.mm(a, b, out=c)) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return out


def alg_counts(T, B, Hq, Hkv, d, W, Bdec, S):
    """Algorithmic FLOPs (QK^T + PV on visible pairs) and bytes (each tensor once)."""
    swa_pairs = W * (W + 1) // 2 + (T - W) * W if T >= W else T * (T + 1) // 2
    glob_pairs = T * (T + 1) // 2
    el = 2  # bf16
    return {
        "swa_flops": 4 * d * swa_pairs * B * Hq,
        "glob_flops": 4 * d * glob_pairs * B * Hq,
        # Q, K, V, G read + O written
        "swa_bytes": B * T * d * el * (3 * Hq + 2 * Hkv),
        "glob_bytes": B * T * d * el * (2 * Hq + 2 * Hkv),
        # K and V cache over [0, pos] + q, k_new, v_new, out
        "gdec_bytes": Bdec * Hkv * S * d * el * 2 + Bdec * d * el * (2 * Hq + 2 * Hkv),
        "sdec_bytes": Bdec * Hkv * W * d * el * 2 + Bdec * d * el * (3 * Hq + 2 * Hkv),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    import global_attention_qk_amd as zg
    from workloads import C4, C5, decode_inputs, prefill_inputs

    dev = "cuda"
    torch.cuda.init()
    if args.only:
        return run_only(args)
    if args.sweep:
        return run_sweep(args)
    if args.configs:
        return run_configs(args)
    if args.model_decode:
        return run_model_decode(args)
    if args.varlen:
        return run_varlen(args)
    if args.backward:
        return run_backward(args)
    T, B, Hq, Hkv, d, W = C4.T, C4.B, C4.Hq, C4.Hkv, C4.d, C4.window
    r = C4.rotary_dim
    # ---- inputs (seeded, generated on the device, outside the timed region) -----------
    q, k, v, g, wq, wk = prefill_inputs(C4, device=dev)
    out_s = torch.empty_like(q)
    out_g = torch.empty_like(q)
    ws_bytes = zg.global_prefill_workspace_bytes(q, k, rotary_dim=r)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    dec = decode_inputs(C5, device=dev)
    Bd, S = C5.B, C5.T
    pos = torch.full((Bd,), S - 1, dtype=torch.int32, device=dev)
    dws = torch.empty(zg.global_decode_workspace_bytes(dec["q"], dec["k_new"], S),
                      dtype=torch.uint8, device=dev)
    out_gd = torch.empty_like(dec["q"])
    out_sd = torch.empty_like(dec["q"])
    torch.cuda.synchronize()

    names = ["swa_prefill", "global_prefill", "global_decode", "swa_decode"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        zg.swa_prefill(q, k, v, g, wq, wk, window=W, rotary_dim=r, out=out_s)
        mark(1)
        zg.global_prefill(q, k, v, wq, wk, rotary_dim=r, workspace=ws, out=out_g)
        mark(2)
        zg.global_decode(dec["q"], dec["k_new"], dec["v_new"], dec["wq"], dec["wk"],
                         dec["k_cache"], dec["v_cache"], pos, rotary_dim=r, workspace=dws,
                         out=out_gd)
        mark(3)
        zg.swa_decode(dec["q"], dec["k_new"], dec["v_new"], dec["g"], dec["wq"], dec["wk"],
                      dec["k_ring"], dec["v_ring"], pos, rotary_dim=r, out=out_sd)
        mark(4)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        print(f"[bench] warmup step {i + 1}/{args.warmup} done", file=sys.stderr, flush=True)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    with ClockSampler() as clock:
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(events[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    per = {n: [] for n in names}
    for ev in events:
        for j, n in enumerate(names):
            per[n].append(ev[j].elapsed_time(ev[j + 1]))
    ms = {n: sum(x) / len(x) for n, x in per.items()}
    ms_step = wall * 1e3 / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_step:.2f} ms/step "
          + " ".join(f"{n}={ms[n]:.3f}ms" for n in names), file=sys.stderr, flush=True)

    cnt = alg_counts(T, B, Hq, Hkv, d, W, Bd, S)
    tokens = B * T + Bd
    value = tokens / (ms_step / 1e3)
    glob_tflops = cnt["glob_flops"] / (ms["global_prefill"] / 1e3) / 1e12
    breakdown = {
        n: {"ms": round(ms[n], 4)} for n in names
    }
    breakdown["swa_prefill"].update(
        tokens_per_s=B * T / (ms["swa_prefill"] / 1e3),
        hbm_GBs=cnt["swa_bytes"] / (ms["swa_prefill"] / 1e3) / 1e9)
    breakdown["swa_prefill"]["hbm_frac"] = breakdown["swa_prefill"]["hbm_GBs"] / PEAK_HBM_GBS
    breakdown["global_prefill"].update(
        tokens_per_s=B * T / (ms["global_prefill"] / 1e3), tflops=glob_tflops,
        mfma_frac=glob_tflops / PEAK_BF16_TFLOPS)
    breakdown["global_decode"].update(
        tokens_per_s=Bd / (ms["global_decode"] / 1e3),
        hbm_GBs=cnt["gdec_bytes"] / (ms["global_decode"] / 1e3) / 1e9)
    breakdown["global_decode"]["hbm_frac"] = breakdown["global_decode"]["hbm_GBs"] / PEAK_HBM_GBS
    breakdown["swa_decode"].update(
        tokens_per_s=Bd / (ms["swa_decode"] / 1e3),
        hbm_GBs=cnt["sdec_bytes"] / (ms["swa_decode"] / 1e3) / 1e9)
    breakdown["prefill_pair_tokens_per_s"] = B * T / ((ms["swa_prefill"] + ms["global_prefill"]) / 1e3)
    breakdown["decode_tokens_per_s"] = Bd / ((ms["global_decode"] + ms["swa_decode"]) / 1e3)

    rec = {
        "metric": "attention tokens/s at 256K ctx (SWA+global prefill, decode); % MFMA/HBM peak",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V/G and caches generated on the device)",
        "config": {
            "workload": "prefill pair (gated SWA W=128 + global causal) B=1 T=262144 "
                        "Hq=32 Hkv=8 d=128 rotary 42 + decode step B=32 ctx=262144",
            "prefill": {"B": B, "T": T, "Hq": Hq, "Hkv": Hkv, "d": d, "window": W,
                        "rotary_dim": r},
            "decode": {"B": Bd, "context": S, "Hq": Hq, "Hkv": Hkv, "d": d, "ring": W},
            "tokens_per_step": tokens,
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "global prefill (causal bf16 MFMA attention, T=262144)",
            "bound": "mfma",
            "achieved": glob_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": glob_tflops / PEAK_BF16_TFLOPS,
            "traffic": measured_traffic(),
            "alg_flops_per_launch": cnt["glob_flops"],
        },
        "breakdown": breakdown,
    }
    # Clock and measured peaks (after the timed steps): the spec peak assumes 2.4 GHz;
    # the fraction at the clock the chip sustained shows what is left for the kernel.
    sclk = clock.report()
    rec["sclk"] = sclk
    del out_s, out_g, ws
    torch.cuda.empty_cache()
    try:
        peaks = measured_peaks()
    except RuntimeError as e:   # e.g. out of memory next to the resident inputs
        peaks = {"error": str(e)[:200]}
    rec["measured_peaks"] = peaks
    if "median_MHz" in sclk:
        at_clock = PEAK_BF16_TFLOPS * sclk["median_MHz"] / 2400.0
        rec["roofline"]["peak_at_sustained_sclk"] = at_clock
        rec["roofline"]["frac_at_sustained_sclk"] = glob_tflops / at_clock
    if "bf16_gemm_TFLOPs" in peaks:
        rec["roofline"]["frac_of_measured_gemm"] = glob_tflops / peaks["bf16_gemm_TFLOPs"]
    if "hbm_copy_GBs" in peaks:
        for n in ("swa_prefill", "global_decode", "swa_decode"):
            breakdown[n]["frac_of_measured_copy"] = breakdown[n]["hbm_GBs"] / peaks["hbm_copy_GBs"]
    if args.cpu_baseline == "on":
        del q, k, v, g
        rec["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def run_model_decode(args):
    """Decode step of the model's 32-layer stack at B=32, context 262,144: 27 gated SWA
    layers (128-slot rings) and 5 global layers (262,144-position caches), each layer with
    its own seeded tensors. Times the batched zgattn_model_decode call and, for reference,
    the same step as 32 single-layer calls. Prints one JSON line."""
    import torch

    import global_attention_qk_amd as zg
    from workloads import C5, STACKS, decode_inputs, stack_kinds

    dev = "cuda"
    kinds = stack_kinds(STACKS["hybrid_5to1"])
    B, S, W, r = C5.B, C5.T, C5.window, C5.rotary_dim
    layers = []
    for i, kind in enumerate(kinds):
        x = decode_inputs(C5, device=dev, layer=i, kind=kind)
        layers.append(dict(kind=kind, q=x["q"], g=x["g"] if kind == "swa" else None,
                           k_new=x["k_new"], v_new=x["v_new"], wq=x["wq"], wk=x["wk"],
                           k_cache=x["k_ring"] if kind == "swa" else x["k_cache"],
                           v_cache=x["v_ring"] if kind == "swa" else x["v_cache"],
                           out=torch.empty_like(x["q"])))
        print(f"[model-decode] layer {i} ({kind}) inputs ready", file=sys.stderr, flush=True)
    pos = torch.full((B,), S - 1, dtype=torch.int32, device=dev)
    ws = torch.empty(zg.model_decode_workspace_bytes(layers, S, rotary_dim=r), dtype=torch.uint8,
                     device=dev)
    dws = torch.empty(zg.global_decode_workspace_bytes(layers[0]["q"], layers[0]["k_new"], S),
                      dtype=torch.uint8, device=dev)

    def batched():
        zg.model_decode(layers, pos, window=W, capacity=S, rotary_dim=r, workspace=ws)

    def per_layer():
        for L in layers:
            if L["kind"] == "swa":
                zg.swa_decode(L["q"], L["k_new"], L["v_new"], L["g"], L["wq"], L["wk"],
                              L["k_cache"], L["v_cache"], pos, rotary_dim=r, out=L["out"])
            else:
                zg.global_decode(L["q"], L["k_new"], L["v_new"], L["wq"], L["wk"],
                                 L["k_cache"], L["v_cache"], pos, rotary_dim=r, workspace=dws,
                                 out=L["out"])

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    swa_layers = [L for L in layers if L["kind"] == "swa"]

    def batched_swa():
        zg.model_decode(swa_layers, pos, window=W, capacity=S, rotary_dim=r, workspace=ws)

    steps = max(args.steps, 1)
    t_b = timed(batched, steps)
    t_l = timed(per_layer, steps)
    t_s = timed(batched_swa, steps)
    n_glob, n_swa = kinds.count("global"), kinds.count("swa")
    el = 2
    glob_bytes = B * C5.Hkv * S * C5.d * el * 2 + B * C5.d * el * (2 * C5.Hq + 2 * C5.Hkv)
    swa_bytes = B * C5.Hkv * W * C5.d * el * 2 + B * C5.d * el * (3 * C5.Hq + 2 * C5.Hkv)
    total = n_glob * glob_bytes + n_swa * swa_bytes
    rec = {
        "model_decode": "32-layer hybrid stack (27 gated SWA, 5 global), B=32, context 262144, "
                        "Hq=32 Hkv=8 d=128 bf16",
        "steps": steps,
        "ms_per_step_batched": t_b,
        "ms_per_step_single_layer_calls": t_l,
        "tokens_per_s": B / (t_b / 1e3),
        "alg_bytes_per_step": total,
        "hbm_GBs": total / (t_b / 1e3) / 1e9,
        "hbm_frac": total / (t_b / 1e3) / 1e9 / PEAK_HBM_GBS,
        "ms_swa_layers_batched": t_s,
        "swa_layers_hbm_GBs": n_swa * swa_bytes / (t_s / 1e3) / 1e9,
        "kv_cache_GiB": (n_glob * B * C5.Hkv * S * C5.d * el * 2 + n_swa * B * C5.Hkv * W * C5.d
                         * el * 2) / 2 ** 30,
    }
    print(json.dumps(rec), flush=True)


def run_backward(args):
    """Backward pass of a gated SWA layer and a global layer at B=1, T=65,536, Hq=32, Hkv=8,
    d=128 (seeded inputs, dout ~ N(0,1)); HIP events around each call (median of the
    steps). FLOPs count the five products of the standard backward (S, dP, dV, dK, dQ) on
    the visible pairs: 2.5x the forward's."""
    import torch

    import global_attention_qk_amd as zg
    from workloads import C3, device_tensor, prefill_inputs, seed_for

    dev = "cuda"
    r, W, T = C3.rotary_dim, C3.window, C3.T
    q, k, v, g, wq, wk = prefill_inputs(C3, device=dev)
    dout = device_tensor(q.shape, seed_for(3, 0, "k_new"), "bf16", dev)
    ws = torch.empty(zg.prefill_backward_workspace_bytes(q, k), dtype=torch.uint8, device=dev)
    cnt = alg_counts(T, C3.B, C3.Hq, C3.Hkv, C3.d, W, 1, 1)
    res = {}
    # "global" hands the forward's row log-sum-exp to the backward (the training path);
    # "global_recompute_lse" lets the backward recompute it
    for kind in ("swa", "global", "global_recompute_lse"):
        gg = g if kind == "swa" else None
        lse = None
        if kind == "swa":
            out = zg.swa_prefill(q, k, v, g, wq, wk, window=W, rotary_dim=r)
        else:
            if kind == "global":
                lse = torch.empty((C3.B, C3.Hq, T), dtype=torch.float32, device=dev)
            out = zg.global_prefill(q, k, v, wq, wk, rotary_dim=r, lse=lse)
        fn = lambda: zg.prefill_backward(q, k, v, gg, wq, wk, out, dout, window=W,
                                         rotary_dim=r, workspace=ws, lse=lse)
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(max(args.steps, 1)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = sorted(ts)[len(ts) // 2]
        flops = 2.5 * cnt["swa_flops" if kind == "swa" else "glob_flops"]
        del out
        res[kind] = {"ms": round(ms, 3), "tokens_per_s": T / (ms / 1e3),
                     "tflops": flops / (ms / 1e3) / 1e12,
                     "mfma_frac": flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS}
        print(f"[backward] {kind}: {ms:.3f} ms", file=sys.stderr, flush=True)
    print(json.dumps({"backward": "B=1 T=65536 Hq=32 Hkv=8 d=128 rotary 42 bf16", **res}),
          flush=True)


def varlen_packings(T: int = 262144):
    """Document lengths of the packed-prefill measurement: 16 equal documents, and 24
    seeded lengths between 1K and 32K tokens rescaled to fill T."""
    import numpy as np
    rng = np.random.default_rng(4242)
    raw = rng.integers(1024, 32768, 24).astype(np.float64)
    lens = np.floor(raw / raw.sum() * T).astype(np.int64)
    lens[-1] += T - lens.sum()
    return {"16x16K": [T // 16] * 16, "24_mixed": [int(x) for x in lens]}


def run_varlen(args):
    """Packed-document prefill of 262,144 tokens (B=1, Hq=32, Hkv=8, d=128, rotary 42,
    W=128): each document attends only within itself, so the global layer's causal work is
    sum(len^2)/2 instead of T^2/2. HIP events around each call (median of the steps)."""
    import numpy as np
    import torch

    import global_attention_qk_amd as zg
    from workloads import C4, prefill_inputs

    dev = "cuda"
    r, W, T = C4.rotary_dim, C4.window, C4.T
    q, k, v, g, wq, wk = prefill_inputs(C4, device=dev)
    q, k, v, g = (x[0] for x in (q, k, v, g))        # packed [T, H, d]
    out = torch.empty_like(q)
    for name, lens in varlen_packings(T).items():
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32,
                          device=dev)
        mx = max(lens)
        ws = torch.empty(zg.global_prefill_varlen_workspace_bytes(q, k, len(lens), rotary_dim=r),
                         dtype=torch.uint8, device=dev)
        calls = {
            "swa": lambda: zg.swa_prefill_varlen(q, k, v, g, wq, wk, cu, mx, window=W,
                                                 rotary_dim=r, out=out),
            "global": lambda: zg.global_prefill_varlen(q, k, v, wq, wk, cu, mx, rotary_dim=r,
                                                       workspace=ws, out=out),
        }
        ms = {}
        for kind, fn in calls.items():
            fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(max(args.steps, 1)):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            ms[kind] = sorted(ts)[len(ts) // 2]
        pairs = sum(n * (n + 1) // 2 for n in lens)
        flops = 4 * C4.d * pairs * C4.Hq
        swa_bytes = T * C4.d * 2 * (3 * C4.Hq + 2 * C4.Hkv)
        rec = {
            "varlen": name, "T": T, "n_docs": len(lens), "max_len": mx,
            "ms": {kd: round(x, 3) for kd, x in ms.items()},
            "tokens_per_s": {kd: T / (x / 1e3) for kd, x in ms.items()},
            "global_tflops": flops / (ms["global"] / 1e3) / 1e12,
            "global_mfma_frac": flops / (ms["global"] / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
            "swa_hbm_frac": swa_bytes / (ms["swa"] / 1e3) / 1e9 / PEAK_HBM_GBS,
        }
        print(json.dumps(rec), flush=True)


SWEEP_T = (4096, 8192, 16384, 32768, 65536, 131072, 262144)


def run_sweep(args):
    """Attention-only stack sweep (B=1, Hq=32, Hkv=8, d=128, rotary 42, W=128): for each
    T, the 32 layers of each stack run back-to-back on one stream over one seeded input
    set (a layer's time does not depend on the values), timed with HIP events around the
    whole stack. Prints one JSON line per T."""
    import torch

    import global_attention_qk_amd as zg
    from workloads import C4, STACKS, prefill_inputs, stack_kinds

    dev = "cuda"
    r, W = C4.rotary_dim, C4.window
    kv_tok = {n: 2 * stack_kinds(p).count("global") * C4.Hkv * C4.d * 2
              for n, p in STACKS.items()}
    Ts = tuple(int(x) for x in args.sweep_t.split(",") if x) or SWEEP_T
    for T in Ts:
        q, k, v, g, wq, wk = prefill_inputs(C4, device=dev, T=T)
        out_s, out_g = torch.empty_like(q), torch.empty_like(q)
        ws = torch.empty(zg.global_prefill_workspace_bytes(q, k, rotary_dim=r),
                         dtype=torch.uint8, device=dev)

        def layer(kind):
            if kind == "swa":
                zg.swa_prefill(q, k, v, g, wq, wk, window=W, rotary_dim=r, out=out_s)
            else:
                zg.global_prefill(q, k, v, wq, wk, rotary_dim=r, workspace=ws, out=out_g)

        def timed(fn, reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            best = []
            for _ in range(reps):
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                best.append(e0.elapsed_time(e1))
            return sorted(best)[len(best) // 2]

        layer("swa")
        layer("global")
        torch.cuda.synchronize()
        reps = 3 if T <= 65536 else 1
        one = {kind: timed(lambda kind=kind: layer(kind), 3) for kind in ("swa", "global")}
        ms = {}
        for name, period in STACKS.items():
            kinds = stack_kinds(period)
            ms[name] = timed(lambda kinds=kinds: [layer(kd) for kd in kinds], reps)
            print(f"[sweep] T={T} {name}: {ms[name]:.2f} ms", file=sys.stderr, flush=True)
        rec = {
            "sweep": "32-layer attention stack, B=1 Hq=32 Hkv=8 d=128 rotary 42 W=128 bf16",
            "T": T,
            "layer_ms": {kd: round(x, 4) for kd, x in one.items()},
            "stack_ms": {n: round(x, 3) for n, x in ms.items()},
            "stack_tokens_per_s": {n: T / (x / 1e3) for n, x in ms.items()},
            "full_over_hybrid": ms["full"] / ms["hybrid_5to1"],
            "full_over_swa_3to1": ms["full"] / ms["swa_3to1"],
            "kv_cache_bytes_per_token": kv_tok,
            "kv_cache_GiB_at_T": {n: x * T / 2 ** 30 for n, x in kv_tok.items()},
        }
        print(json.dumps(rec), flush=True)
        del q, k, v, g, out_s, out_g, ws
        torch.cuda.empty_cache()


# Targets of the measurement table: (configuration, layer) -> ms per call.
CONFIG_TARGETS_MS = {
    ("C2", "swa"): 0.0979, ("C2", "global"): 0.440,
    ("C3", "swa"): 0.392, ("C3", "global"): 28.15, ("C3", "stack"): 151.3,
    ("C4", "swa"): 1.566, ("C4", "global"): 450.4,
    ("C5", "global_decode"): 7.16, ("C5", "swa_decode_batched_per_layer"): 0.0037,
}


def run_configs(args):
    """The measurement table's configurations, each call timed on its own: 5 untimed
    warm-ups, then >= 20 timed calls (>= 5 for the 256K global layer and the 32-layer
    stack), with a 1 GiB buffer written before every call so that neither L2 nor the
    256 MB Infinity Cache still holds the inputs; HIP events around the call only. Prints
    one JSON line per (configuration, layer) with median, min and p90, tokens/s, the
    roofline fraction and the target.

    The default flush reads the 1 GiB buffer (a sum over it), which evicts the inputs just
    as a write does but leaves clean lines behind. A written buffer leaves up to 256 MB of
    dirty lines in the memory-side cache, and their write-back (about 32 us at 8 TB/s) is
    then charged to the next call: a plain read of 453 MB takes about 25 % longer after a
    write flush than after a read flush, which matters for the microsecond decode calls
    and not for the millisecond prefill layers. The flush also keeps the GPU busy while
    the host prepares the measured call, so that the first event does not time the host."""
    import torch

    import global_attention_qk_amd as zg
    from workloads import C1, C2, C3, C4, C5, STACKS, decode_inputs, prefill_inputs, stack_kinds

    dev = "cuda"
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    if args.flush == "read":
        evict = lambda: torch.sum(flush, dim=0, out=sink)
    else:
        evict = lambda: flush.fill_(7.0)

    def timed(fn, reps):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            evict()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ts.sort()
        return ts

    def emit(cfg, layer, ts, tokens, bound, work):
        med = ts[len(ts) // 2]
        rec = {"config": cfg, "layer": layer, "flush": args.flush, "reps": len(ts),
               "median_ms": med,
               "min_ms": ts[0], "p90_ms": ts[min(len(ts) - 1, (9 * len(ts)) // 10)],
               "tokens_per_s": tokens / (med / 1e3) if tokens else None}
        if bound == "mfma":
            rec.update(bound="mfma", achieved_TFLOPs=work / (med / 1e3) / 1e12,
                       frac=work / (med / 1e3) / 1e12 / PEAK_BF16_TFLOPS)
        elif bound == "hbm":
            rec.update(bound="hbm", achieved_GBs=work / (med / 1e3) / 1e9,
                       frac=work / (med / 1e3) / 1e9 / PEAK_HBM_GBS)
        tgt = CONFIG_TARGETS_MS.get((cfg, layer))
        if tgt is not None:
            rec.update(target_ms=tgt, met=med <= tgt)
        print(json.dumps(rec), flush=True)

    def pair(cfg, wl, reps_swa, reps_glob, T=None):
        T = wl.T if T is None else T
        q, k, v, g, wq, wk = prefill_inputs(wl, device=dev, T=T)
        r, W = wl.rotary_dim, wl.window
        out = torch.empty_like(q)
        cnt = alg_counts(T, wl.B, wl.Hq, wl.Hkv, wl.d, W, 1, 1)
        ts = timed(lambda: zg.swa_prefill(q, k, v, g, wq, wk, window=W, rotary_dim=r, out=out),
                   reps_swa)
        emit(cfg, "swa", ts, wl.B * T, "hbm", cnt["swa_bytes"])
        if reps_glob:
            ws = torch.empty(zg.global_prefill_workspace_bytes(q, k, rotary_dim=r),
                             dtype=torch.uint8, device=dev)
            ts = timed(lambda: zg.global_prefill(q, k, v, wq, wk, rotary_dim=r, workspace=ws,
                                                 out=out), reps_glob)
            emit(cfg, "global", ts, wl.B * T, "mfma", cnt["glob_flops"])
            return q, k, v, g, wq, wk, out, ws
        return None

    # C1: fp32 gated SWA layer (parity configuration; launch-bound)
    q, k, v, g, wq, wk = prefill_inputs(C1, device=dev)
    out = torch.empty_like(q)
    ts = timed(lambda: zg.swa_prefill(q, k, v, g, wq, wk, window=C1.window,
                                      rotary_dim=C1.rotary_dim, out=out), 20)
    emit("C1", "swa", ts, C1.B * C1.T, None, 0)
    # C2, C4: the layer pair
    pair("C2", C2, 20, 20)
    # C3: both layer kinds at T=65536 and the 32-layer hybrid stack over one input set
    held = pair("C3", C3, 20, 5)
    q, k, v, g, wq, wk, out, ws = held
    kinds = stack_kinds(STACKS["hybrid_5to1"])

    def stack():
        for kd in kinds:
            if kd == "swa":
                zg.swa_prefill(q, k, v, g, wq, wk, window=C3.window, rotary_dim=C3.rotary_dim,
                               out=out)
            else:
                zg.global_prefill(q, k, v, wq, wk, rotary_dim=C3.rotary_dim, workspace=ws,
                                  out=out)
    emit("C3", "stack", timed(stack, 5), C3.T, None, 0)
    del q, k, v, g, out, ws, held
    torch.cuda.empty_cache()
    pair("C4", C4, 20, 5)
    torch.cuda.empty_cache()
    # C5: decode, B=32 at context 262144
    dec = decode_inputs(C5, device=dev)
    S, W, r = C5.T, C5.window, C5.rotary_dim
    pos = torch.full((C5.B,), S - 1, dtype=torch.int32, device=dev)
    cnt = alg_counts(1, 1, C5.Hq, C5.Hkv, C5.d, W, C5.B, S)
    dws = torch.empty(zg.global_decode_workspace_bytes(dec["q"], dec["k_new"], S),
                      dtype=torch.uint8, device=dev)
    out = torch.empty_like(dec["q"])
    ts = timed(lambda: zg.global_decode(dec["q"], dec["k_new"], dec["v_new"], dec["wq"],
                                        dec["wk"], dec["k_cache"], dec["v_cache"], pos,
                                        rotary_dim=r, workspace=dws, out=out), 20)
    emit("C5", "global_decode", ts, C5.B, "hbm", cnt["gdec_bytes"])
    ts = timed(lambda: zg.swa_decode(dec["q"], dec["k_new"], dec["v_new"], dec["g"], dec["wq"],
                                     dec["wk"], dec["k_ring"], dec["v_ring"], pos,
                                     rotary_dim=r, out=out), 20)
    emit("C5", "swa_decode", ts, C5.B, "hbm", cnt["sdec_bytes"])
    del dec
    torch.cuda.empty_cache()
    # the 27 gated SWA layers of a model decode step in one launch (per-layer time)
    swa_layers = []
    for i in range(27):
        x = decode_inputs(C5, device=dev, layer=i, kind="swa")
        swa_layers.append(dict(kind="swa", q=x["q"], g=x["g"], k_new=x["k_new"],
                               v_new=x["v_new"], wq=x["wq"], wk=x["wk"], k_cache=x["k_ring"],
                               v_cache=x["v_ring"]))
    ts = timed(lambda: zg.model_decode(swa_layers, pos, window=W, rotary_dim=r), 20)
    emit("C5", "swa_decode_batched_per_layer", [t / 27 for t in ts], C5.B, "hbm",
         cnt["sdec_bytes"])
    # context for the line above: a library read (torch.sum) of the 27 layers' ring bytes
    ring_bytes = sum(x["k_cache"].numel() * x["k_cache"].element_size() * 2
                     for x in swa_layers)
    del swa_layers
    buf = torch.ones(ring_bytes // 4, dtype=torch.float32, device=dev)
    out0 = torch.empty((), dtype=torch.float32, device=dev)
    ts = timed(lambda: torch.sum(buf, dim=0, out=out0), 20)
    emit("C5", "plain_read_of_27_rings", ts, 0, "hbm", ring_bytes)


def run_only(args):
    """One call kind alone, warmup + steps launches (for rocprofv3 runs)."""
    import torch

    import global_attention_qk_amd as zg
    from workloads import C4, C5, decode_inputs, prefill_inputs

    dev = "cuda"
    r, W = C4.rotary_dim, C4.window
    if args.only == "copy":
        n = 1 << 30
        x = torch.randint(0, 255, (n,), dtype=torch.uint8, device=dev)
        y = torch.empty_like(x)
        call = lambda: y.copy_(x)
    elif args.only in ("swa_prefill", "global_prefill"):
        from workloads import C2
        wl = C2 if args.workload == "c2" else C4
        q, k, v, g, wq, wk = prefill_inputs(wl, device=dev, gated=args.only == "swa_prefill")
        out = torch.empty_like(q)
        if args.only == "swa_prefill":
            call = lambda: zg.swa_prefill(q, k, v, g, wq, wk, window=W, rotary_dim=r, out=out)
        elif args.fused_k:
            call = lambda: zg.global_prefill(q, k, v, wq, wk, rotary_dim=r, workspace=None,
                                             out=out)
        else:
            ws = torch.empty(zg.global_prefill_workspace_bytes(q, k, rotary_dim=r),
                             dtype=torch.uint8, device=dev)
            call = lambda: zg.global_prefill(q, k, v, wq, wk, rotary_dim=r, workspace=ws, out=out)
    else:
        dec = decode_inputs(C5, device=dev)
        S = C5.T
        pos = torch.full((C5.B,), S - 1, dtype=torch.int32, device=dev)
        out = torch.empty_like(dec["q"])
        if args.only == "global_decode":
            dws = torch.empty(zg.global_decode_workspace_bytes(dec["q"], dec["k_new"], S),
                              dtype=torch.uint8, device=dev)
            call = lambda: zg.global_decode(dec["q"], dec["k_new"], dec["v_new"], dec["wq"],
                                            dec["wk"], dec["k_cache"], dec["v_cache"], pos,
                                            rotary_dim=r, workspace=dws, out=out)
        else:
            call = lambda: zg.swa_decode(dec["q"], dec["k_new"], dec["v_new"], dec["g"],
                                         dec["wq"], dec["wk"], dec["k_ring"], dec["v_ring"], pos,
                                         rotary_dim=r, out=out)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    print(f"[bench] {args.only}: {args.steps} launches, "
          f"{e0.elapsed_time(e1) / max(args.steps, 1):.3f} ms each", flush=True)


def _host_facts():
    """CPU model and the BLAS library numpy calls (name, version, threads)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        import numpy  # noqa: F401  (loads the BLAS library that threadpoolctl inspects)
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = (f"{libs[0].get('internal_api')} {libs[0].get('version')} "
                    f"({libs[0].get('architecture')})")
    except Exception:
        pass
    return model, blas


def cpu_baseline(budget_s: float, n_rows: int = 512):
    """The fp64 oracle on a bounded sample of the same workload, scaled to tokens/s.

    Sample: ``n_rows`` stratified query rows of the T=262144 prefill pair (rows 0..15,
    window edges, tile boundaries, T-1, the rest uniform; all 32 heads; the global rows
    read every key up to the row, the SWA rows only their window) and one decode sequence
    of each kind at context 262144. A global row costs in proportion to the keys it sees
    (i + 1), so its measured time is scaled by T(T+1)/2 / sum(i + 1) over the sample; an
    SWA row by the layer's visible pairs / sum(min(i + 1, W)); decode by B = 32.
    """
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import attn as O
    from workloads import C4, C5, decode_inputs, prefill_inputs, stratified_rows

    cores = min(len(os.sched_getaffinity(0)), 16)
    T, W = C4.T, C4.window
    q, k, v, g, wq, wk = prefill_inputs(C4, device="cuda")
    f = lambda t: t.float().cpu().numpy()
    rows = stratified_rows(T, n_rows, 7, W)
    kh, vh = f(k), f(v)
    qh, gh = f(q[:, rows]), f(g[:, rows])
    wqh, wkh = f(wq), f(wk)
    del q, k, v, g
    t0 = time.perf_counter()
    O.prefill_rows(qh, kh, vh, None, wqh, wkh, rows, rotary_dim=C4.rotary_dim, threads=cores)
    t_glob = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.prefill_rows(qh, kh, vh, gh, wqh, wkh, rows, window=W, rotary_dim=C4.rotary_dim,
                   threads=cores)
    t_swa = time.perf_counter() - t0
    del kh, vh
    glob_scale = (T * (T + 1) / 2) / float(np.sum(rows + 1))
    swa_pairs = W * (W + 1) // 2 + (T - W) * W
    swa_scale = swa_pairs / float(np.sum(np.minimum(rows + 1, W)))
    dec = decode_inputs(C5, device="cuda", B=1)
    dh = {n: f(t) for n, t in dec.items()}
    S = C5.T
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        O.decode_global(dh["q"], dh["k_new"], dh["v_new"], dh["wq"], dh["wk"], dh["k_cache"],
                        dh["v_cache"], np.array([S - 1]), rotary_dim=C5.rotary_dim)
        t_gd = time.perf_counter() - t0
        t0 = time.perf_counter()
        O.decode_swa(dh["q"], dh["k_new"], dh["v_new"], dh["g"], dh["wq"], dh["wk"],
                     dh["k_ring"], dh["v_ring"], np.array([S - 1]), window=C5.window,
                     rotary_dim=C5.rotary_dim)
        t_sd = time.perf_counter() - t0
    step_s = t_glob * glob_scale + t_swa * swa_scale + C5.B * (t_gd + t_sd)
    model, blas = _host_facts()
    return {
        "value": (T + C5.B) / step_s,
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{len(rows)} stratified query rows of the T=262144 prefill pair (all 32 "
                  f"heads; global {t_glob:.2f} s for {int(np.sum(rows + 1))} visible keys per "
                  f"head, scaled by pairs x{glob_scale:.0f}; SWA {t_swa:.2f} s, x{swa_scale:.0f})"
                  f" and one decode sequence per layer kind at context 262144 (global "
                  f"{t_gd:.2f} s, SWA {t_sd:.4f} s, x32), summed to one step of 262144 "
                  f"prefill + 32 decode tokens",
        "seconds_per_step_estimate": step_s,
        "seconds_by_layer": {"global_prefill": t_glob * glob_scale,
                             "swa_prefill": t_swa * swa_scale,
                             "global_decode": C5.B * t_gd, "swa_decode": C5.B * t_sd},
        "cpu_model": model,
        "blas": blas,
        "threads": cores,
        "parallel_jobs_prefill": min(cores, C4.B * C4.Hkv),
    }


if __name__ == "__main__":
    main()
