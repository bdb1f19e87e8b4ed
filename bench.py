#!/usr/bin/env python3
"""Benchmark of the routed-MoE expert layer on one MI355X.

A step is one moe_forward: dispatch -> gate-up grouped GEMM + SiLU epilogue ->
down grouped GEMM -> weighted combine, over one batch of synthetic input that
is already resident in HBM.  The default workload is the Mixtral-style layer
(8 experts, top-2, hidden 4096, intermediate 14336, 4096 tokens); --config
selects another workload of the same family (see workloads.CONFIGS).

Printed (one JSON line): expert-compute TFLOP/s of the layer (value), µs per
layer (mean, median, p10, p90), HBM GB/s, the stages timed alone
(stages_us: dispatch, expert compute, combine, and for the softmax-routed
workloads the router top-k ahead of dispatch, alone and fused into the
dispatch kernels), the roofline of the dominant
kernel (the gate-up grouped GEMM, timed alone with HIP events on the stream it
is launched on), and the CPU oracle timed on a bounded sample of the same
workload.  The decode workloads cycle 32 routing draws (seeds 1000..1031) one
per step, with value and GB/s = sum of work / sum of time, so that draws that
touch fewer experts (or none) count their time.  static_capacity adds
`replays`: 50 HIP-graph replays, each with a device token count
T_i ~ U{1..T}, with median/p10/p90 µs and the per-replay fraction of the
binding roof.

With the default workload the same line also carries `per_config`: every
other full-size workload measured in the same run, each with µs/layer, its
binding-roof fraction (and MFMA / HBM fractions beside it) and the gate-up
kernel's own roofline: the 96-of-384 decode shares T = 1, 8, 32, 128 (cold:
L2/MALL evicted before each step, 32 routing draws cycled; each also timed
as replays of the layer recorded as a HIP graph, `graph_replay`, and at T = 1
through the single-launch forward, `single_launch`), the prefill
shares T = 2048, 8192 with uniform routing (seeds 0-2) and Zipf s = 1.2
routing (seeds 0-4, reported per seed), a supplementary T = 16384 point of
the same shape (seed 0, labelled `supplementary`), and the static-capacity layer (50
HIP-graph replays with a device token count T_i ~ U{1..2048}, and the full
buffer called eagerly).  --no-per-config leaves it out.

Algorithmic work (what the method must do, not what an implementation moves):
  F = 6*H*I*R flop, R = valid dispatched rows (2*H*2I gate-up + 2*I*H down per row)
  B = 6*H*I*n_touched + 2*H*T (x) + 2*H*T (out) + 8*T*K (ids, weights) bytes
  gate-up kernel: F_gu = 4*H*I*R flop,
                  B_gu = 4*H*I*n_touched (weights) + 2*H*R (rows read) + 2*I*R (h written)
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import statistics
import sys
import time

REPO = os.path.dirname(os.path.abspath(__file__))
if REPO not in sys.path:
    sys.path.insert(0, REPO)

METRIC = "µs/MoE layer + expert-compute TFLOPS (and HBM GB/s) vs roofline, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense BF16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)

DESCR = {
    "tiny": "tiny: 8 experts, top-2, hidden 256, intermediate 512, 64 tokens",
    "mixtral": "mixtral-style: 8 experts, top-2, hidden 4096, intermediate 14336, 4096 tokens",
}


def describe(cfg):
    if cfg.name in DESCR:
        return DESCR[cfg.name]
    routing = {"ep_uniform": "uniform", "ep_zipf": f"zipf s={cfg.zipf_s}",
               "softmax_topk": "softmax top-k"}[cfg.routing]
    return (f"{cfg.name}: {cfg.num_experts} local of {cfg.pool} experts, top-{cfg.top_k}, "
            f"hidden {cfg.hidden}, intermediate {cfg.intermediate}, {cfg.num_tokens} tokens, "
            f"{routing} routing")


def pmc_traffic(kernel_key: str, src_hash: str, units: int, seed: int = 0, hint: int = 0):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when there is none for this kernel/workload, the kernel sources changed
    since the counters were taken, the plan was forced (the counters are of the
    automatic plan) or the entry is of another routing seed."""
    if hint != 0:
        return None
    path = os.path.join(REPO, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        data = json.load(fh)
    ent = data.get(kernel_key)
    if not ent or ent.get("src_sha256") != src_hash:
        return None
    if ent.get("seed") is not None and ent["seed"] != seed:
        return None
    return ent.get("bytes_per_launch")


# The sources the grouped-GEMM kernels are compiled from: a change to their
# code (not to their comments) voids the committed counter figures; host-side
# API code does not.
GEMM_SOURCES = ("moe_gemm.hip", "moe_internal.h")


def _code_only(text: str) -> str:
    """The source with comments and layout removed: a comment edit leaves the
    kernels, and so the counter figures, unchanged."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_src_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(REPO, "mixture_experts_routed_02_amd", "csrc")
    for name in GEMM_SOURCES:
        with open(os.path.join(csrc, name), encoding="utf-8") as fh:
            h.update(name.encode() + b"\0" + _code_only(fh.read()).encode())
    return h.hexdigest()


def cpu_baseline(inp_host, wgu, wd, cfg, budget_tokens: int, mx=None, fmt="bf16"):
    """The oracle, as it stands, on the first `budget_tokens` tokens (with
    mx = (codes_gu, scales_gu, codes_d, scales_d) on the MX weights of fmt)."""
    import numpy as np
    import torch

    import oracle

    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    toks = np.arange(min(budget_tokens, cfg.num_tokens))
    ids = inp_host["topk_ids"].numpy()
    used = sorted({int(e) for e in ids[toks].reshape(-1) if 0 <= e < cfg.num_experts})

    def bits(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    class Experts:
        def __init__(self, w):
            self.host = {e: (w[e].cpu().numpy() if w.dtype == torch.uint8 else bits(w[e].cpu()))
                         for e in used}
            self.n = w.shape[0]

        def __len__(self):
            return self.n

        def __getitem__(self, e):
            return self.host[int(e)]

    xg = bits(inp_host["x"])
    if mx is None:
        wug, wdg = Experts(wgu), Experts(wd)
        t0 = time.perf_counter()
        oracle.forward_tokens(xg, ids, inp_host["topk_weights"].numpy(), wug, wdg, toks)
    else:
        qs = [Experts(t) for t in mx]
        t0 = time.perf_counter()
        fwd = oracle.forward_tokens_mxfp8 if fmt == "mxfp8" else oracle.forward_tokens_mxfp4
        fwd(xg, ids, inp_host["topk_weights"].numpy(), *qs, toks)
    dt = time.perf_counter() - t0
    rows = int(((ids[toks] >= 0) & (ids[toks] < cfg.num_experts)).sum())
    flops = 6.0 * cfg.hidden * cfg.intermediate * rows
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:  # pragma: no cover
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"first {len(toks)} tokens of the same inputs ({rows} expert rows), "
                      f"float64 numpy, {dt:.1f} s",
            "host": {"nproc": os.cpu_count(), "cpu_model": model}}


# ---------------------------------------------------------------------------
# per_config: the other full-size workloads, measured in the same run
# ---------------------------------------------------------------------------
PER_CONFIG = (
    ("ep_decode_T1", "decode"), ("ep_decode_T8", "decode"), ("ep_decode_T32", "decode"),
    ("ep_decode_T128", "decode"),
    ("ep_prefill_T2048", "prefill"), ("ep_prefill_T8192", "prefill"),
    ("ep_prefill_T2048_zipf", "prefill"), ("ep_prefill_T8192_zipf", "prefill"),
    ("static_capacity", "static"),
    ("ep_prefill_T16384", "prefill"),   # supplementary: ~256 rows per expert
)
SUPPLEMENTARY = {"ep_prefill_T16384": "supplementary point of the EP prefill shape at 16384 tokens "
                                      "(about 256 rows per local expert): one weight pass allows "
                                      "up to 78.5% of the MFMA peak here"}
PREFILL_SEED_OVERRIDE = {"ep_prefill_T16384": (0,)}
DECODE_DRAWS = 32          # routing draws (seeds 1000..1031), one per step
PREFILL_SEEDS = {"ep_uniform": (0, 1, 2), "ep_zipf": (0, 1, 2, 3, 4)}
PREFILL_STEPS = 10         # timed calls per seed


def _layer_work(ids_h, E, H, I, K, t_valid):
    """(F, B, R, n_touched): algorithmic flop and bytes of one layer call."""
    import torch
    v = ids_h[:t_valid]
    v = v[(v >= 0) & (v < E)]
    r = int(v.numel())
    n_t = int(torch.unique(v).numel()) if r else 0
    return 6.0 * H * I * r, 6.0 * H * I * n_t + 4.0 * H * t_valid + 8.0 * t_valid * K, r, n_t


def _roof(F, B, sec):
    mf = F / sec / 1e12 / PEAK_BF16_TFLOPS
    hf = B / sec / 1e9 / PEAK_HBM_GBPS
    binding = "mfma" if F / max(B, 1.0) >= RIDGE else "hbm"
    return {"binding": binding, "binding_frac": mf if binding == "mfma" else hf,
            "mfma_frac": mf, "hbm_frac": hf}


def per_config_sweep(dev, kernel_reps: int):
    """Measure every workload of PER_CONFIG (see the module docstring)."""
    import torch

    import mixture_experts_routed_02_amd as moe
    from mixture_experts_routed_02_amd import ops
    import workloads as W

    stream = torch.cuda.current_stream(dev)
    scratch = torch.ones((1 << 29,), dtype=torch.float16, device=dev)   # 1 GiB

    def evict():
        scratch.max()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def timed_us(call, reps, cold):
        """Event-timed µs per call (mean); short calls wait behind a spin so
        that the events see the GPU's time, not the host's."""
        call()
        torch.cuda.synchronize()
        evs = [(ev(), ev()) for _ in range(reps)]
        torch.cuda._sleep(5_000_000)
        for a, b in evs:
            if cold:
                evict()
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        return statistics.fmean(a.elapsed_time(b) for a, b in evs) * 1e3

    out_all = {}
    weights = {}
    for name, kind in PER_CONFIG:
        cfg = W.CONFIGS[name]
        T, K, E, H, I = cfg.num_tokens, cfg.top_k, cfg.num_experts, cfg.hidden, cfg.intermediate
        key = (E, H, I)
        if key not in weights:
            weights.clear()
            torch.cuda.empty_cache()
            weights[key] = W.make_weights(cfg, 0, dev)
        wgu, wd = weights[key]
        p = moe.problem(T, K, E, H, I, cfg.capacity)
        ws = ops.make_workspace(p, dev)
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        off = torch.empty((E + 1,), dtype=torch.int32, device=dev)
        if kind == "decode":
            seeds = [1000 + d for d in range(DECODE_DRAWS)]
        elif kind == "prefill":
            seeds = list(PREFILL_SEED_OVERRIDE.get(name, PREFILL_SEEDS[cfg.routing]))
        else:
            seeds = [0]
        routes = []
        for sd in seeds:
            ids_h, w_h = W.make_routing(cfg, sd)
            x_d = W.make_x(cfg, sd if kind == "prefill" else 0).to(dev)
            routes.append((sd, ids_h, x_d, ids_h.to(dev), w_h.to(dev)))
        cold = kind == "decode"

        def call(i, nt=None):
            _, _, x_d, ids_d, w_d = routes[i % len(routes)]
            ops.forward(p, x_d, ids_d, w_d, wgu, wd, num_tokens_dev=nt, expert_offsets=off,
                        out=out, workspace=ws)

        steps = len(routes) * (1 if kind == "decode" else PREFILL_STEPS)
        for i in range(max(len(routes), 5)):
            call(i)
        torch.cuda.synchronize()
        evs = [(ev(), ev()) for _ in range(steps)]
        for i, (a, b) in enumerate(evs):
            if cold:
                evict()
            a.record(stream)
            call(i)
            b.record(stream)
        torch.cuda.synchronize()
        us = [a.elapsed_time(b) * 1e3 for a, b in evs]
        work = [_layer_work(r[1], E, H, I, K, T) for r in routes]
        F = sum(work[i % len(routes)][0] for i in range(steps))
        B = sum(work[i % len(routes)][1] for i in range(steps))
        sec = sum(us) * 1e-6
        ent = {"us_per_layer": statistics.fmean(us), "us_median": statistics.median(us),
               "tflops": F / sec / 1e12, "hbm_gbps": B / sec / 1e9, **_roof(F, B, sec),
               "steps": steps, "timing": ("cold: L2/MALL evicted before each step; "
                                          f"{len(routes)} routing draws cycled" if cold else
                                          f"back-to-back, {PREFILL_STEPS} calls per seed, "
                                          f"seeds {seeds}"),
               "valid_rows_mean": statistics.fmean(w_[2] for w_ in work),
               "experts_touched_mean": statistics.fmean(w_[3] for w_ in work)}
        if kind == "decode":
            # the same draws, cold, through (a) replays of the layer recorded as
            # a HIP graph (no host launch gaps) and (b) the single-launch
            # forward where it applies (T*K <= 8, I % 1024 == 0)
            ids_c, w_c = routes[0][3].clone(), routes[0][4].clone()
            g = ops.MoEGraph(p, routes[0][2], ids_c, w_c, wgu, wd, expert_offsets=off, out=out,
                             workspace=ws)

            def replay(i):
                ids_c.copy_(routes[i % len(routes)][3])
                w_c.copy_(routes[i % len(routes)][4])
                return g.launch

            def single(i):
                _, _, x_d, ids_d, w_d = routes[i % len(routes)]
                return lambda: ops.forward_single(p, x_d, ids_d, w_d, wgu, wd, expert_offsets=off,
                                                  out=out, workspace=ws)

            variants = [("graph_replay", replay)]
            if T * K <= 8 and I % 1024 == 0:
                variants.append(("single_launch", single))
            for vname, prep in variants:
                for i in range(len(routes)):
                    prep(i)()
                torch.cuda.synchronize()
                vev = [(ev(), ev()) for _ in range(steps)]
                for i, (a, b) in enumerate(vev):
                    fn = prep(i)
                    evict()
                    a.record(stream)
                    fn()
                    b.record(stream)
                torch.cuda.synchronize()
                vus = [a.elapsed_time(b) * 1e3 for a, b in vev]
                ent[vname] = {"us_per_layer": statistics.fmean(vus),
                              "us_median": statistics.median(vus),
                              **_roof(F, B, sum(vus) * 1e-6)}
            g.close()
            if len(variants) > 1:
                ent["single_launch"]["barrier_timeouts"] = ops.single_launch_status()
        if kind == "prefill":
            per_seed = []
            for j, (sd, ids_h, _, _, _) in enumerate(routes):
                us_j = [us[i] for i in range(steps) if i % len(routes) == j]
                F_j, B_j, R_j, n_j = work[j]
                v = ids_h[(ids_h >= 0)]
                cnt = torch.bincount(v.reshape(-1).long(), minlength=cfg.pool)
                ent_j = {"seed": sd, "us_per_layer": statistics.fmean(us_j),
                         **_roof(F_j, B_j, statistics.fmean(us_j) * 1e-6),
                         "valid_rows": R_j, "experts_touched": n_j,
                         "max_rows_per_local_expert": int(cnt[:E].max())}
                if cfg.routing == "ep_zipf":
                    ent_j["most_popular_expert_is_local"] = bool(int(cnt.argmax()) < E)
                per_seed.append(ent_j)
            ent["per_seed"] = per_seed
        # the dominant kernel alone: gate-up grouped GEMM + SiLU epilogue (first route)
        _, ids_h0, x0, ids0, _ = routes[0]
        x_disp, off2, _, _ = ops.dispatch(p, x0, ids0)
        hbuf = torch.empty((p.capacity or T * K, I), dtype=torch.bfloat16, device=dev)
        gu_us = timed_us(lambda: ops.gate_up(p, x_disp, off2, wgu, h=hbuf), kernel_reps, cold)
        _, _, R0, n0 = work[0]
        F_gu = 4.0 * H * I * R0
        B_gu = 4.0 * H * I * n0 + 2.0 * H * R0 + 2.0 * I * R0
        if F_gu / max(B_gu, 1.0) >= RIDGE:
            gu = {"bound": "mfma", "achieved": F_gu / (gu_us * 1e-6) / 1e12, "unit": "TFLOP/s",
                  "peak": PEAK_BF16_TFLOPS}
        else:
            gu = {"bound": "hbm", "achieved": B_gu / (gu_us * 1e-6) / 1e9, "unit": "GB/s",
                  "peak": PEAK_HBM_GBPS}
        gu.update({"frac": gu["achieved"] / gu["peak"], "avg_launch_us": gu_us,
                   "algorithmic_flop": F_gu, "algorithmic_bytes": B_gu,
                   "route": f"seed {routes[0][0]}", "cold": cold})
        ent["gate_up"] = gu
        del x_disp, hbuf
        if kind == "static":
            # HIP-graph replays with a device token count T_i ~ U{1..T}
            _, ids_h, x_d, ids_d, w_d = routes[0]
            ntok = torch.full((1,), T, dtype=torch.int32, device=dev)
            g = ops.MoEGraph(p, x_d, ids_d, w_d, wgu, wd, num_tokens_dev=ntok, expert_offsets=off,
                             out=out, workspace=ws)
            t_i = W.make_static_token_counts(0, W.STATIC_REPLAYS, T)
            for _ in range(3):
                g.launch()
            torch.cuda.synchronize()
            rev = [(ev(), ev()) for _ in t_i]
            for (a, b), tv in zip(rev, t_i):
                ntok.fill_(tv)
                a.record(stream)
                g.launch()
                b.record(stream)
            torch.cuda.synchronize()
            rus = [a.elapsed_time(b) * 1e3 for a, b in rev]
            fr = []
            for tv, u in zip(t_i, rus):
                f_i, b_i, _, _ = _layer_work(ids_h, E, H, I, K, tv)
                fr.append(max(f_i / (PEAK_BF16_TFLOPS * 1e12), b_i / (PEAK_HBM_GBPS * 1e9))
                          / (u * 1e-6))
            q = statistics.quantiles(rus, n=10, method="inclusive")
            ent["replays"] = {"n": len(t_i), "tokens_min": min(t_i), "tokens_max": max(t_i),
                              "us_median": statistics.median(rus), "us_p10": q[0],
                              "us_p90": q[8], "binding_frac_median": statistics.median(fr),
                              "binding_frac_min": min(fr), "binding_frac_max": max(fr)}
            g.close()
        ent["workload"] = describe(cfg)
        if name in SUPPLEMENTARY:
            ent["supplementary"] = SUPPLEMENTARY[name]
        out_all[name] = ent
        del routes, ws, out, off
        torch.cuda.synchronize()
    del weights, scratch
    torch.cuda.empty_cache()
    return out_all


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="mixtral")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--hint", type=int, default=0, help="grouped-GEMM plan (0 auto, 1-4 forced)")
    ap.add_argument("--cold", action="store_true",
                    help="read a 1 GiB buffer before each step (outside the timed events) so "
                         "the weights come from HBM, not L2/MALL")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the layer recorded as a HIP graph (moe_graph_*)")
    ap.add_argument("--kernel-reps", type=int, default=10)
    ap.add_argument("--draws", type=int, default=None,
                    help="routing draws cycled one per step (seeds 1000, 1001, ...; default 32 "
                         "for the decode workloads, else 1 = the --seed routing)")
    ap.add_argument("--replays", type=int, default=None,
                    help="extra: HIP-graph replays with a device token count T_i ~ U{1..T} "
                         "(default 50 for static_capacity, else 0)")
    ap.add_argument("--cpu-tokens", type=int, default=None,
                    help="tokens in the oracle's timed sample (default by workload)")
    ap.add_argument("--weights", choices=("bf16", "mxfp8", "mxfp4"), default="bf16",
                    help="expert weight format: bf16, MXFP8 (e4m3 codes + one e8m0 scale per 32 "
                         "values) or MXFP4 (e2m1 codes, two per byte, same scales), quantized on "
                         "the device before timing")
    ap.add_argument("--packed", action="store_true",
                    help="expert weights (bf16) or codes (MX) in the skinny pack layout, packed "
                         "on the device before timing; the skinny plan serves every batch size")
    ap.add_argument("--tiled-packed", action="store_true",
                    help="expert weights (bf16) or MX codes in the tiled pack layout (packed on "
                         "the device before timing); the tiled plans serve every batch size")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="leave out the per_config sweep over the other workloads")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark measures the single-GPU expert path; "
                          "runs on more than one GPU are not part of it", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import mixture_experts_routed_02_amd as moe
    from mixture_experts_routed_02_amd import ops
    import workloads as W

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    moe.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = W.CONFIGS[args.config]
    T, K, E, H, I = cfg.num_tokens, cfg.top_k, cfg.num_experts, cfg.hidden, cfg.intermediate

    x_h = W.make_x(cfg, args.seed)
    ids_h, w_h = W.make_routing(cfg, args.seed)
    wgu, wd = W.make_weights(cfg, args.seed, dev)
    x, ids, w = x_h.to(dev), ids_h.to(dev), w_h.to(dev)
    mx = args.weights in ("mxfp8", "mxfp4")
    packed = args.packed
    tpacked = args.tiled_packed
    if tpacked and (packed or args.graph or args.replays):
        raise SystemExit("--tiled-packed is a layout of its own, for eager launches")
    if tpacked and not mx:
        tgu, td = ops.tiled_pack(wgu), ops.tiled_pack(wd)
        torch.cuda.synchronize()
    if packed and not mx:
        if args.graph or args.replays:
            raise SystemExit("--graph / --replays record the row-major layer; use --weights bf16")
        pgu, pd = ops.skinny_pack(wgu, True), ops.skinny_pack(wd, False)
        torch.cuda.synchronize()
    if mx:
        if args.graph or args.replays:
            raise SystemExit("--graph / --replays record the bf16 layer; use --weights bf16")
        qgu, sgu = ops.mx_quantize(wgu, args.weights)
        qd, sd = ops.mx_quantize(wd, args.weights)
        if packed:
            qgu, qd = ops.mx_pack(qgu, True, args.weights), ops.mx_pack(qd, False, args.weights)
        if tpacked:   # the tiled (prefill) pack layout of the codes
            qgu, qd = ops.mx_tiled_pack(qgu, args.weights), ops.mx_tiled_pack(qd, args.weights)
        torch.cuda.synchronize()
    # HBM bytes per weight value: bf16, or a code (1 or 1/2 byte) plus 1/32 of a scale byte
    wbytes = {"bf16": 2.0, "mxfp8": 1.0 + 1.0 / 32.0, "mxfp4": 0.5 + 1.0 / 32.0}[args.weights]
    draws = args.draws if args.draws is not None else (32 if cfg.name.startswith("ep_decode") else 1)
    if draws > 1:   # routing draws cycled one per step, same x and weights
        routes_h = [W.make_routing(cfg, 1000 + d) for d in range(draws)]
        routes = [(i_h.to(dev), w_h_.to(dev)) for i_h, w_h_ in routes_h]
    else:
        routes_h, routes = [(ids_h, w_h)], [(ids, w)]
    p = moe.problem(T, K, E, H, I, cfg.capacity, args.hint)
    ws = ops.make_workspace(p, dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    off = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    scratch = torch.ones((1 << 29,), dtype=torch.float16, device=dev) if args.cold else None

    def evict():
        # a read-only sweep: leaves L2/MALL full of clean lines of another buffer
        if scratch is not None:
            scratch.max()

    graph = None
    if args.graph:
        graph = ops.MoEGraph(p, x, ids, w, wgu, wd, expert_offsets=off, out=out, workspace=ws)

    if args.graph and draws > 1:
        raise SystemExit("--graph replays one recorded routing; use --draws 1")

    def step(i=0):
        if graph is not None:
            graph.launch()
        else:
            ri, rw = routes[i % draws]
            if mx:
                ops.forward_mx(p, x, ri, rw, qgu, sgu, qd, sd, args.weights, expert_offsets=off,
                               out=out, workspace=ws, packed=packed, tiled_packed=tpacked)
            elif packed:
                ops.forward_packed(p, x, ri, rw, pgu, pd, expert_offsets=off, out=out,
                                   workspace=ws)
            elif tpacked:
                ops.forward_tiled_packed(p, x, ri, rw, tgu, td, expert_offsets=off, out=out,
                                         workspace=ws)
            else:
                ops.forward(p, x, ri, rw, wgu, wd, expert_offsets=off, out=out, workspace=ws)

    def work(ids_t, t_valid):
        # algorithmic flop and bytes of one layer call (host copy of the routing)
        v = ids_t[:t_valid]
        v = v[(v >= 0) & (v < E)]
        r = int(v.numel())
        n_touched = int(torch.unique(v).numel()) if r else 0
        return (6.0 * H * I * r, 3.0 * wbytes * H * I * n_touched + 4.0 * H * t_valid + 8.0 * t_valid * K,
                r, n_touched)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    F, B, R, touched = work(ids_h, T)                 # the --seed routing (draw 0 if draws == 1)
    FB = [work(i_h, T) for i_h, _ in routes_h]
    F_steps = sum(FB[i % draws][0] for i in range(args.steps))
    B_steps = sum(FB[i % draws][1] for i in range(args.steps))

    # ---- timed region: exactly `steps` layer calls ------------------------
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evict()
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in ev]          # ms
    ms_step = statistics.fmean(per) if args.cold else wall * 1e3 / args.steps
    sec = ms_step / 1e3
    pct = statistics.quantiles(per, n=10, method="inclusive") if len(per) > 1 else per * 9

    def timed(call):
        """Mean event-timed ms of `call` over --kernel-reps calls (an eviction
        read before each under --cold).  Calls shorter than the host's launch
        latency are enqueued behind a bounded spin kernel, so that the events
        see the GPU's time rather than the host's."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        short = e0.elapsed_time(e1) < 0.3
        sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.kernel_reps)]
        if short:
            torch.cuda._sleep(5_000_000)
        for a, b in sev:
            evict()
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        return statistics.fmean(a.elapsed_time(b) for a, b in sev)

    # ---- dominant kernel alone: the gate-up grouped GEMM ------------------
    x_disp, off2, _, _ = ops.dispatch(p, x, ids)
    hbuf = torch.empty((p.capacity or T * K, I), dtype=torch.bfloat16, device=dev)
    if mx:
        gu_call = lambda: ops.gate_up_mx(p, x_disp, off2, qgu, sgu, args.weights, h=hbuf,
                                         packed=packed, tiled_packed=tpacked)
    elif packed:
        gu_call = lambda: ops.gate_up_packed(p, x_disp, off2, pgu, h=hbuf)
    elif tpacked:
        gu_call = lambda: ops.gate_up_tiled_packed(p, x_disp, off2, tgu, h=hbuf)
    else:
        gu_call = lambda: ops.gate_up(p, x_disp, off2, wgu, h=hbuf)
    gu_call()
    k_ms = timed(gu_call)

    # ---- the stages alone (same inputs, --seed routing) -------------------
    x_disp_s, off_s, row_src_s, token_row_s = ops.dispatch(p, x, ids, workspace=ws)
    y_s = ops.expert_compute(p, x_disp_s, off_s, wgu, wd, workspace=ws)
    out_s = torch.empty_like(out)
    stage_calls = {
        "dispatch": lambda: ops.dispatch(p, x, ids, workspace=ws,
                                         out=(x_disp_s, off_s, row_src_s, token_row_s)),
        "expert_compute": lambda: ops.expert_compute(p, x_disp_s, off_s, wgu, wd, workspace=ws,
                                                     y_disp=y_s),
        "combine": lambda: ops.combine(p, y_s, token_row_s, w, out=out_s),
    }
    if mx or packed or tpacked:   # the staged MX / packed calls: the gate-up grouped GEMM alone
        del stage_calls["expert_compute"]
        stage_calls["gate_up"] = gu_call
    if cfg.routing == "softmax_topk":   # the router step ahead of dispatch, on the same seed's logits
        logits = W.make_logits(cfg, args.seed).to(dev)
        ids_r = torch.empty_like(ids)
        w_r = torch.empty_like(w)
        stage_calls = {"router": lambda: ops.router_topk(p, logits, topk_ids=ids_r, topk_weights=w_r),
                       **stage_calls}
        # the router fused into the dispatch kernels (one launch fewer)
        stage_calls["router_dispatch"] = lambda: ops.router_dispatch(
            p, logits, x, topk_ids=ids_r, topk_weights=w_r, workspace=ws,
            out=(x_disp_s, off_s, row_src_s, token_row_s))
    # long calls first: the spin that short calls sit behind lowers the clock
    # for a while after it
    order = ["expert_compute", "gate_up", "combine", "dispatch", "router_dispatch", "router"]
    stages_us = {name: timed(stage_calls[name]) * 1e3 for name in order if name in stage_calls}

    F_gu = 4.0 * H * I * R
    B_gu = 2.0 * wbytes * H * I * touched + 2.0 * H * R + 2.0 * I * R
    mfma_bound = (F_gu / max(B_gu, 1.0)) >= RIDGE
    # the host plan rule of the library: forced hint, else rows per expert T*K/E
    rpe = T * K / E
    kind = args.hint if args.hint in (1, 2, 3, 4) else (1 if rpe <= 24 else 2 if rpe <= 96 else 4)
    if packed:
        kind = 1
    if tpacked and kind == 1:
        kind = 2
    kernel_name = "gemm_skinny_kernel" if kind == 1 else "gemm_tiled_kernel"
    if mx:
        wf = 8 if args.weights == "mxfp8" else 4
        kernel_name = f"gemm_skinny_mx_kernel<{wf}>" if kind == 1 else f"gemm_tiled_kernel<MXFP{wf}>"
    if packed:
        kernel_name += " (packed weights)"
    if tpacked:
        kernel_name += " (tiled pack layout)"
    traffic = pmc_traffic(f"{kernel_name}<gated>@{cfg.name}", kernel_src_hash(), 1, args.seed,
                          args.hint)
    if mfma_bound:
        ach = F_gu / (k_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / PEAK_BF16_TFLOPS, "traffic": traffic}
    else:
        ach = B_gu / (k_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBPS, "traffic": traffic}
    roof.update({"kernel": f"{kernel_name} (gate-up + SiLU epilogue)", "avg_launch_us": k_ms * 1e3,
                 "algorithmic_flop": F_gu, "algorithmic_bytes": B_gu})

    # ---- extra: graph replays with a device token count T_i ~ U{1..T} -----
    n_rep = args.replays if args.replays is not None else (
        50 if cfg.name == "static_capacity" and not mx else 0)
    replays = None
    if n_rep > 0:
        ntok = torch.empty((1,), dtype=torch.int32, device=dev)
        ntok.fill_(T)
        g = ops.MoEGraph(p, x, ids, w, wgu, wd, num_tokens_dev=ntok, expert_offsets=off,
                         out=out, workspace=ws)
        t_i = W.make_static_token_counts(args.seed, n_rep, T)
        rev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_rep)]
        for _ in range(3):
            g.launch()
        torch.cuda.synchronize()
        for (a, b), tv in zip(rev, t_i):
            ntok.fill_(tv)        # a fill kernel on the same stream, outside the events
            evict()
            a.record(stream)
            g.launch()
            b.record(stream)
        torch.cuda.synchronize()
        rus = [a.elapsed_time(b) * 1e3 for a, b in rev]
        fr = []
        for tv, us in zip(t_i, rus):
            f_i, b_i, _, _ = work(ids_h, tv)
            fr.append(max(f_i / (PEAK_BF16_TFLOPS * 1e12), b_i / (PEAK_HBM_GBPS * 1e9)) / (us * 1e-6))
        q = statistics.quantiles(rus, n=10, method="inclusive")
        replays = {"n": n_rep, "tokens_min": min(t_i), "tokens_max": max(t_i),
                   "us_median": statistics.median(rus), "us_p10": q[0], "us_p90": q[8],
                   "roof_frac_median": statistics.median(fr), "roof_frac_min": min(fr),
                   "roof_frac_max": max(fr),
                   "note": "binding-roof fraction per replay: max(F_i/MFMA peak, B_i/HBM peak)/t_i"}
        g.close()

    total = sec * args.steps
    result = {
        "metric": METRIC,
        "value": F_steps / total / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "us_per_layer": ms_step * 1e3,
        "us_per_layer_median": statistics.median(per) * 1e3,
        "us_per_layer_p10": pct[0] * 1e3,
        "us_per_layer_p90": pct[8] * 1e3,
        "hbm_gbps": B_steps / total / 1e9,
        "layer_roofline": {"mfma_frac": F_steps / total / 1e12 / PEAK_BF16_TFLOPS,
                           "hbm_frac": B_steps / total / 1e9 / PEAK_HBM_GBPS,
                           "binding": "mfma" if F_steps / max(B_steps, 1.0) >= RIDGE else "hbm"},
        "stages_us": stages_us,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": describe(cfg), "tokens": T, "top_k": K, "experts": E,
                   "global_experts": cfg.pool, "hidden": H, "intermediate": I,
                   "capacity": p.capacity or T * K, "valid_rows": R, "experts_touched": touched,
                   "routing_draws": draws,
                   "valid_rows_mean": statistics.fmean(fb[2] for fb in FB),
                   "experts_touched_mean": statistics.fmean(fb[3] for fb in FB),
                   "seed": args.seed, "timing": ("cold (L2/MALL evicted per step)" if args.cold
                                                 else "back-to-back")
                   + (", HIP graph replay" if args.graph else ", eager launches"),
                   "kernel_hint": args.hint,
                   "packed": packed, "tiled_packed": tpacked,
                   "weights": {"bf16": "bf16",
                               "mxfp8": "mxfp8: e4m3 codes + one e8m0 scale per 32 values along K",
                               "mxfp4": "mxfp4: e2m1 codes (two per byte) + one e8m0 scale per "
                                        "32 values along K"}[args.weights]},
        "roofline": roof,
    }
    if replays is not None:
        result["replays"] = replays
    if not args.no_cpu_baseline:
        budget = args.cpu_tokens
        if budget is None:
            budget = {"mixtral": T, "tiny": 64}.get(cfg.name, max(16, min(T, 64)))
        result["cpu_baseline"] = cpu_baseline({"x": x_h, "topk_ids": ids_h, "topk_weights": w_h},
                                              wgu, wd, cfg, budget,
                                              (qgu, sgu, qd, sd) if mx else None, args.weights)
    sweep = (cfg.name == "mixtral" and not args.no_per_config and not mx and not packed
             and not tpacked and not args.graph and args.hint == 0)
    if sweep:
        del x_disp, hbuf, x_disp_s, y_s, out_s, wgu, wd, ws, out, scratch
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        result["per_config"] = per_config_sweep(dev, args.kernel_reps)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
